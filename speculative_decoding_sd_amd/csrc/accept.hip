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
//   accept_rowpart   one block per slice of a logits row (rows x slices
//                    blocks): the slice's argmax (smallest id on ties),
//                    finiteness and, for sampled rows, its max and fp64
//                    mass sum exp((l - max)/T)
//   accept_rowmerge  one wave per row: merges the slices into the row max m,
//                    argmax, Z = sum exp((l-m)/T) and p_t of the row's draft
//   accept_topp_*    sampled rows with top_p < 1: the nucleus threshold
//                    lambda (exact: all tokens tied with the last kept logit
//                    are kept), the kept mass, p_t of the draft
//   accept_plan      one wave per request: the sequential accept decision
//   accept_draw_*    the fp64 inverse-CDF draw of a sampled final token: one
//                    pass over the drawn row in (request, slice) blocks sums
//                    each 512-id chunk, then one block per request scans the
//                    chunk sums and walks the crossing chunk
//   accept_pack      exclusive scan of emitted counts, packed tokens
// Statistics and running sums that decide integers are fp64 and reduced in a
// fixed order, so results do not depend on scheduling.
#include <math.h>

#include <algorithm>
#include <mutex>

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
    int relaxed_ok; // relaxed rule: the draft this row judges survives
    int pad;
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

// exp(y) for y <= 0 in fp64, table-driven (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989): y = (64k + j) ln2/64 + r with
// |r| <= ln2/128, exp(y) = 2^k 2^(j/64) e^r.  r comes from a two-part
// (Cody-Waite) reduction with fused multiply-adds; e^r - 1 is its degree-5
// Taylor polynomial (truncation below r^6/720 < 4e-17).  tab[j] = 2^(j/64)
// from exp2 (see exp_table_init).  About 12 fp64 operations against ~40 for a
// general exp; accuracy within about 2 ulp.
constexpr double kExpInvL = 0x1.71547652b82fep+6;   // 64 / ln 2
constexpr double kExpLHi = 0x1.62e42fefa39efp-7;    // ln 2 / 64, leading double
constexpr double kExpLLo = 0x1.abc9e3b39803fp-62;   // ln 2 / 64 - kExpLHi
// The two halves of exp_neg, for callers that batch the table reads.
// y is clamped to -746 first (max ignores NaN), which maps y <= -746, -inf
// and NaN to 2^-1077 * [1, 2) scaled by ldexp: 0 after rounding.  For
// -746 < y <= -708 the result is the rounded subnormal.
struct ExpRed {
    double p;  // e^r - 1
    int ni;    // n = 64k + j
};
__device__ __forceinline__ ExpRed exp_reduce(double y) {
    ExpRed q;
    const double yc = __builtin_fmax(y, -746.0);
    const double n = __builtin_rint(yc * kExpInvL);
    double r = __builtin_fma(-n, kExpLHi, yc);
    r = __builtin_fma(-n, kExpLLo, r);
    q.p = r * (1.0 + r * (0.5 + r * (1.0 / 6.0 + r * (1.0 / 24.0 + r * (1.0 / 120.0)))));
    q.ni = (int)n;
    return q;
}
__device__ __forceinline__ double exp_finish(const ExpRed& q, double tj) {
    return __builtin_amdgcn_ldexp(__builtin_fma(tj, q.p, tj), q.ni >> 6);
}
__device__ __forceinline__ double exp_neg(double y, const double* tab) {
    const ExpRed q = exp_reduce(y);
    return exp_finish(q, tab[q.ni & 63]);
}

// LDS table 2^(j/64), j = 0..63, for exp_neg; a block's first 64 threads fill
// it (the caller synchronises before use).
__device__ __forceinline__ void exp_table_init(double* tab) {
    if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
}

// exp((x - m) / T) in fp64, with 1/T precomputed once per row.
__device__ __forceinline__ double tempered(float x, float m, double invT, const double* tab) {
    return exp_neg(((double)x - (double)m) * invT, tab);
}

// Per-thread accumulator over a slice of one row: the running max (its
// smallest id), finiteness, and for sampled rows z = sum exp((x - best)/T)
// over the thread's elements, rescaled whenever best rises.
struct RowAcc {
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    bool nonfinite = false, anyfin = false;
    double z = 0.0;
    int beat = 0;  // relaxed rows: elements ranked before the draft
};

// Folds N elements into a, in the thread's visit order (ids rise along it).
// The group max decides everything but the sum: finiteness (a NaN, or a
// max of +inf), whether a value above -inf was seen, and whether best rises;
// only then is the group searched for the first id of its max and z
// rescaled.  Sampled rows then add the group's terms eight at a time (all
// eight table reads issued before the first is used) as pairwise trees.
// FAST (sampled rows without a nucleus): each term is exp2 in float32 of
// (x - best) * log2(e) / T, eight of them summed in float32, the group sums
// accumulated in fp64.  A term is then within a few float32 ulps, so Z is
// within about 1e-6 relative: Z of such a row only scales p_t of the draft
// (an acceptance decision it could move lies within 1e-6 of u) and the
// draw's weights (a common scale, which the draw's running sums cancel).
// Rows with a nucleus keep fp64 terms: their threshold compares the kept
// mass with top_p * Z.
// RELAX rows also count the elements ranked before the draft d (logit xd)
// in the order (logit desc, id asc).
template <bool STOCH, bool RELAX, bool FAST, int N>
__device__ __forceinline__ void row_fold(RowAcc& a, const float (&x)[N], const int (&v)[N],
                                         double invT, const double* tab, float xd, int d,
                                         float k2) {
    if constexpr (RELAX) {
#pragma unroll
        for (int e = 0; e < N; ++e) a.beat += (x[e] > xd) | ((x[e] == xd) & (v[e] < d));
    }
    float gm = x[0];
    bool nan = x[0] != x[0];
#pragma unroll
    for (int e = 1; e < N; ++e) {
        gm = fmaxf(gm, x[e]);
        nan |= x[e] != x[e];
    }
    a.nonfinite |= nan | (gm == INFINITY);
    a.anyfin |= gm > -INFINITY;
    if (gm > a.best) {
        int id = v[N - 1];
#pragma unroll
        for (int e = N - 1; e >= 0; --e) id = x[e] == gm ? v[e] : id;
        if constexpr (STOCH) a.z *= exp_neg(((double)a.best - (double)gm) * invT, tab);
        a.best = gm;
        a.bidx = id;
    }
    if constexpr (STOCH && FAST) {
        constexpr int G = N < 8 ? N : 8;
        const float mt = a.best;
        double acc = 0.0;
#pragma unroll
        for (int g = 0; g < N; g += G) {
            float w[G];
#pragma unroll
            for (int e = 0; e < G; ++e)  // max drops the NaN of -inf - -inf (term 0)
                w[e] = __builtin_amdgcn_exp2f(fmaxf((x[g + e] - mt) * k2, -160.f));
#pragma unroll
            for (int h = 1; h < G; h <<= 1)
#pragma unroll
                for (int e = 0; e + h < G; e += 2 * h) w[e] += w[e + h];
            acc += (double)w[0];
        }
        a.z += acc;
    } else if constexpr (STOCH) {
        constexpr int G = N < 8 ? N : 8;
        const double mtd = (double)a.best;
        double acc = 0.0;
#pragma unroll
        for (int g = 0; g < N; g += G) {
            ExpRed q[G];
            double tj[G], w[G];
#pragma unroll
            for (int e = 0; e < G; ++e) q[e] = exp_reduce(((double)x[g + e] - mtd) * invT);
#pragma unroll
            for (int e = 0; e < G; ++e) tj[e] = tab[q[e].ni & 63];
#pragma unroll
            for (int e = 0; e < G; ++e) w[e] = exp_finish(q[e], tj[e]);
#pragma unroll
            for (int h = 1; h < G; h <<= 1)
#pragma unroll
                for (int e = 0; e + h < G; e += 2 * h) w[e] += w[e + h];
            acc += w[0];
        }
        a.z += acc;
    }
}

// One pass over ids [v_lo, v_hi) of a row (v_lo a multiple of the vector
// width when vec_ok); U vectors in flight per thread.  k2 = log2(e) / T in
// float32 (FAST rows).
template <typename T, bool STOCH, bool RELAX, bool FAST = false>
__device__ __forceinline__ void row_pass(const T* lr, int v_lo, int v_hi, bool vec_ok, RowAcc& a,
                                         double invT, const double* tab, float xd, int d,
                                         float k2 = 0.f) {
    constexpr int E = Logit<T>::kPerVec;
    constexpr int U = RELAX ? 2 : 4;  // vectors in flight (fewer with the rank count)
    int v0 = v_lo;
    if (vec_ok) {
        const int c_lo = v_lo / E, c_hi = v_hi / E;
        int c = c_lo + (int)threadIdx.x;
        for (; c + (U - 1) * 256 < c_hi; c += U * 256) {
            u32x4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = *(const u32x4*)(lr + (size_t)(c + u * 256) * E);
            float x[U * E];
            int v[U * E];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    x[u * E + e] = Logit<T>::lane(w[u], e);
                    v[u * E + e] = (c + u * 256) * E + e;
                }
            row_fold<STOCH, RELAX, FAST>(a, x, v, invT, tab, xd, d, k2);
        }
        for (; c < c_hi; c += 256) {
            const u32x4 w = *(const u32x4*)(lr + (size_t)c * E);
            float x[E];
            int v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                x[e] = Logit<T>::lane(w, e);
                v[e] = c * E + e;
            }
            row_fold<STOCH, RELAX, FAST>(a, x, v, invT, tab, xd, d, k2);
        }
        v0 = c_hi * E;
    }
    for (int vv = v0 + (int)threadIdx.x; vv < v_hi; vv += 256) {
        const float x[1] = {Logit<T>::at(lr, vv)};
        const int v[1] = {vv};
        row_fold<STOCH, RELAX, FAST>(a, x, v, invT, tab, xd, d, k2);
    }
}

// Statistics of one slice of a row, merged over slices by accept_rowmerge.
struct RowPart {
    float best;   // slice max (-inf if none finite)
    int bidx;     // its smallest id
    int bits;     // 1: a NaN or +inf seen; 2: a value above -inf seen
    int beat;     // relaxed rows: elements of the slice ranked before the draft
    double z;     // sum over the slice of exp((x - best)/T) (sampled and relaxed rows)
};

// Grid: rows x splits blocks of 256 threads; block (row, s) covers ids
// [s*span, min(V, (s+1)*span)) of its row.  Relaxed greedy rows (top-N > 0)
// take the sum at T = 1 and count the elements ranked before their draft
// (compiled in only for launches with relaxed parameters, RX).
template <typename T, bool RX>
__global__ __launch_bounds__(256) void accept_rowpart(const T* __restrict__ logits,
                                                      const int32_t* __restrict__ drafts,
                                                      const float* __restrict__ temperature,
                                                      const float* __restrict__ top_p,
                                                      const int32_t* __restrict__ relaxed_topk,
                                                      RowPart* __restrict__ parts, int Q, int V,
                                                      int splits, int span, int vec_ok) {
    __shared__ double s_exptab[64];
    __shared__ float s_best[4];
    __shared__ int s_idx[4], s_beat[4];
    __shared__ double s_z[4];
    exp_table_init(s_exptab);
    __syncthreads();
    const int row = blockIdx.x / splits, sp = blockIdx.x - row * splits;
    const int b = row / Q;
    const T* lr = logits + (size_t)row * V;
    const int v_lo = sp * span, v_hi = min(V, v_lo + span);
    const int i = row - b * Q, K = Q - 1;
    const float Tb = temperature[b];
    const bool relaxed = RX && Tb == 0.f && relaxed_topk[b] > 0;
    const double invT = Tb > 0.f ? 1.0 / (double)Tb : 1.0;
    const int d = (relaxed && i < K) ? drafts[(size_t)b * K + i] : -1;
    const bool count = d >= 0 && d < V;
    const bool stoch = Tb > 0.f || count;  // the slice's sum is needed
    const float xd = count ? Logit<T>::at(lr, d) : 0.f;
    const bool vk = vec_ok != 0;
    // Sampled rows without a nucleus take float32 terms (see row_fold).
    const bool fast = Tb > 0.f && !count && (top_p == nullptr || !(top_p[b] < 1.f));
    RowAcc a;
    if (count) row_pass<T, true, RX>(lr, v_lo, v_hi, vk, a, invT, s_exptab, xd, d);
    else if (fast)
        row_pass<T, true, false, true>(lr, v_lo, v_hi, vk, a, invT, s_exptab, xd, d,
                                       (float)(1.4426950408889634 * invT));
    else if (stoch) row_pass<T, true, false>(lr, v_lo, v_hi, vk, a, invT, s_exptab, xd, d);
    else row_pass<T, false, false>(lr, v_lo, v_hi, vk, a, invT, s_exptab, xd, d);
    float best = a.best;
    int bidx = a.bidx;
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
    const int nonfinite = __syncthreads_or(a.nonfinite);
    const int anyfin = __syncthreads_or(a.anyfin);
    best = s_best[0];
    bidx = s_idx[0];
    for (int w = 1; w < 4; ++w)
        if (s_best[w] > best || (s_best[w] == best && s_idx[w] < bidx)) {
            best = s_best[w];
            bidx = s_idx[w];
        }
    double z = 0.0;
    if (stoch && !nonfinite && best > -INFINITY) {
        // The threads' (best, z) pairs rescaled to the slice max, summed by a
        // fixed-order wave butterfly, then over the waves in order.
        double zt = a.z * exp_neg(((double)a.best - (double)best) * invT, s_exptab);
        zt = wave_sum(zt);
        if (lane == 0) s_z[wave] = zt;
        __syncthreads();
        z = ((s_z[0] + s_z[1]) + s_z[2]) + s_z[3];
    }
    int beat = 0;
    if (count) {
        int bt = a.beat;
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) bt += shfl_xor(bt, msk);
        if (lane == 0) s_beat[wave] = bt;
        __syncthreads();
        beat = (s_beat[0] + s_beat[1]) + (s_beat[2] + s_beat[3]);
    }
    if (threadIdx.x == 0) {
        RowPart p;
        p.best = best;
        p.bidx = bidx;
        p.bits = (nonfinite ? 1 : 0) | (anyfin ? 2 : 0);
        p.beat = beat;
        p.z = z;
        parts[blockIdx.x] = p;
    }
}

// One wave per row, a lane per slice (at most 64): merges the row's slices
// (max, smallest id on ties, Z = sum_s z_s exp((best_s - m)/T) reduced by a
// fixed butterfly), checks the request's parameters and, for sampled rows
// that judge a draft, p_t of that draft.  Relaxed rows ([TRT-MTP] "寬松接受"):
// the draft survives when fewer than N tokens rank before it and its
// probability exp(l_d - m)/Z (T = 1) is not below the top-1 probability 1/Z
// minus delta, i.e. exp(l_d - m) >= 1 - delta Z.
template <typename T>
__global__ __launch_bounds__(256) void accept_rowmerge(
    const T* __restrict__ logits, const int32_t* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ top_p, int has_probs,
    const int32_t* __restrict__ relaxed_topk, const float* __restrict__ relaxed_delta,
    const RowPart* __restrict__ parts, RowStat* __restrict__ stats, int rows, int K, int V,
    int splits) {
    __shared__ double s_exptab[64];
    exp_table_init(s_exptab);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int Q = K + 1, b = row / Q, i = row - b * Q;
    const float Tb = temperature[b];
    const float tp = top_p ? top_p[b] : 1.f;
    const bool stoch = Tb > 0.f;
    const int rN = relaxed_topk ? relaxed_topk[b] : 0;
    const bool relaxed = Tb == 0.f && rN > 0;
    const double delta = (relaxed && relaxed_delta) ? (double)relaxed_delta[b] : 0.0;
    const int d = (i < K) ? drafts[(size_t)b * K + i] : -1;
    const T* lr = logits + (size_t)row * V;
    const float xd = (d >= 0 && d < V) ? Logit<T>::at(lr, d) : 0.f;
    int flags = 0;
    if (isnan(Tb) || Tb < 0.f) flags |= SD_DERR_PARAM;
    if (stoch && (isnan(tp) || tp <= 0.f || (!has_probs && K > 0))) flags |= SD_DERR_PARAM;
    if (rN < 0) flags |= SD_DERR_PARAM;
    if (relaxed && (!relaxed_delta || !(delta >= 0.0) || isinf(delta))) flags |= SD_DERR_PARAM;
    RowPart p;
    p.best = -INFINITY;
    p.bidx = 0x7fffffff;
    p.bits = 0;
    p.beat = 0;
    p.z = 0.0;
    if (lane < splits) p = parts[(size_t)row * splits + lane];
    float best = p.best;
    int bidx = p.bidx, bits = p.bits, beat = p.beat;
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
        const float ob = shfl_xor(best, msk);
        const int oi = shfl_xor(bidx, msk);
        if (ob > best || (ob == best && oi < bidx)) {
            best = ob;
            bidx = oi;
        }
        bits |= shfl_xor(bits, msk);
        beat += shfl_xor(beat, msk);
    }
    if ((bits & 1) || !(bits & 2)) flags |= SD_DERR_NONFINITE;
    double z = 0.0, pt_d = 0.0;
    int relaxed_ok = 0;
    if (stoch && !flags) {
        const double invT = 1.0 / (double)Tb;
        const double zt = lane < splits
            ? p.z * exp_neg(((double)p.best - (double)best) * invT, s_exptab) : 0.0;
        z = wave_sum(zt);
        if (d >= 0 && d < V) pt_d = tempered(xd, best, invT, s_exptab) / z;
    } else if (relaxed && !flags && i < K && d >= 0 && d < V) {
        const double zt = lane < splits
            ? p.z * exp_neg((double)p.best - (double)best, s_exptab) : 0.0;
        z = wave_sum(zt);
        const double e_d = exp_neg((double)xd - (double)best, s_exptab);
        relaxed_ok = beat < rN && e_d >= 1.0 - delta * z;
    }
    if (lane == 0) {
        RowStat st;
        st.m = best;
        st.lambda = -INFINITY;
        st.argmax = bidx;
        st.flags = flags;
        st.zkeep = z;
        st.pt_d = pt_d;
        st.relaxed_ok = relaxed_ok;
        st.pad = 0;
        stats[row] = st;
    }
}

// ---------------------------------------------------------------------------
// Nucleus threshold for bf16 rows.  One block of 1024 threads per row walks
// the 65536 orderable bf16 keys down from the row maximum in windows of 8192:
// an exact u32 count per key (LDS atomics, four 16-byte loads in flight per
// thread), the mass of each level = count * exp((value - m) / T), a
// fixed-order prefix over levels (per thread over its 8 levels, then a lane
// scan per wave, then the 16 waves in order) until the running mass reaches
// top_p * Z.  The level where it does is lambda; every token with logit >=
// lambda is kept.
// ---------------------------------------------------------------------------
constexpr int kWin = 8192;
constexpr int kToppThreads = 1024;
constexpr int kToppLevels = kWin / kToppThreads;  // levels per thread

__global__ __launch_bounds__(kToppThreads) void accept_topp_bf16(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ top_p,
    RowStat* __restrict__ stats, int K, int V, int vec_ok) {
    __shared__ double s_exptab[64];
    exp_table_init(s_exptab);
    __syncthreads();
    extern __shared__ __attribute__((aligned(16))) uint32_t s_hist[];  // kWin
    __shared__ double s_wtot[kToppThreads / 64];
    __shared__ int s_found, s_lkey;
    __shared__ double s_zkeep, s_cum;
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double cum = 0.0;  // mass above the current window
    int lkey = -1;
    double zkeep = st.zkeep;
    for (int top = (int)bf16_key(__float_as_uint(m) >> 16);; top -= kWin) {
        const int bottom = top - (kWin - 1) > 0 ? top - (kWin - 1) : 0;
        for (int w = tid; w < kWin; w += kToppThreads) s_hist[w] = 0;
        __syncthreads();
        auto count = [&](uint32_t bits16) {
            const int k = (int)bf16_key(bits16);
            if (k <= top && k >= bottom) atomicAdd(&s_hist[top - k], 1u);
        };
        int v0 = 0;
        if (vec_ok) {
            const int nvec = V / 8;
            int c = tid;
            for (; c + 3 * kToppThreads < nvec; c += 4 * kToppThreads) {
                u32x4 w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) w[u] = *(const u32x4*)(lr + (size_t)(c + u * kToppThreads) * 8);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e) count((w[u][e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
            for (; c < nvec; c += kToppThreads) {
                const u32x4 w = *(const u32x4*)(lr + (size_t)c * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) count((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
            v0 = nvec * 8;
        }
        for (int v = v0 + tid; v < V; v += kToppThreads) count(lr[v]);
        __syncthreads();
        // Thread t owns levels [8 t, 8 t + 8) of the window, highest first.
        double mass[kToppLevels];
        double part = 0.0;
#pragma unroll
        for (int j = 0; j < kToppLevels; ++j) {
            const int idx = tid * kToppLevels + j;
            const uint32_t c = s_hist[idx];
            mass[j] = (c && top - idx >= bottom)
                ? (double)c * tempered(bf16_to_f32(key_to_bf16(top - idx)), m, invT, s_exptab)
                : 0.0;
            part += mass[j];
        }
        // Exclusive prefix of the threads' parts in thread order: a lane scan
        // per wave, then the waves in order (offset by the mass above).
        double incl = part;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        double excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.0;
        if (lane == 63) s_wtot[wave] = incl;
        if (tid == 0) s_found = 0;
        __syncthreads();
        // pre of thread t+1 is nxt of thread t bit for bit (same additions),
        // so exactly one thread sees the crossing.
        double wpre = cum;
        for (int w = 0; w < wave; ++w) wpre += s_wtot[w];
        const double pre = wpre + excl, nxt = wpre + incl;
        if (pre < target && nxt >= target) {
            double run = pre;
            int last = -1;
            double at_last = pre;
            for (int j = 0; j < kToppLevels; ++j) {
                const int idx = tid * kToppLevels + j;
                if (!s_hist[idx] || top - idx < bottom) continue;
                run += mass[j];
                last = top - idx;
                at_last = run;
                if (run >= target) break;
            }
            s_lkey = last;
            s_zkeep = at_last;
            s_found = 1;
        }
        if (tid == kToppThreads - 1) s_cum = nxt;
        __syncthreads();
        if (s_found) {
            lkey = s_lkey;
            zkeep = s_zkeep;
            break;
        }
        cum = s_cum;
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
            if (xd >= out.lambda) out.pt_d = tempered(xd, m, invT, s_exptab) / out.zkeep;
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
    __shared__ double s_exptab[64];
    exp_table_init(s_exptab);
    __syncthreads();
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
            if (f32_key(__float_as_uint(x)) >= mid) part += tempered(x, m, invT, s_exptab);
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
        if (d >= 0 && d < V && lr[d] >= out.lambda) out.pt_d = tempered(lr[d], m, invT, s_exptab) / out.zkeep;
        stats[row] = out;
    }
}

enum { kModeInvalid = 0, kModeDone = 1, kModeResidual = 2, kModeTarget = 3, kModeTree = 4 };

// ---------------------------------------------------------------------------
// Per-request decision and final-token draw, spread over the chip:
//   accept_plan       one wave per request, a lane per draft: the sequential
//                     accept decision from the row statistics (greedy,
//                     relaxed, rejection or tree); every output but a sampled
//                     final token; the plan of the draw
//   accept_draw_w     (request, slice) blocks, sampled final tokens: one fp64
//                     pass over the drawn row, per 512-id chunk the sums the
//                     draw needs (below)
//   accept_draw_pick  one block per sampled request: the chunks' weight sums,
//                     a fixed-order scan of them to the chunk whose running
//                     sum first exceeds u * total, then the token inside it
// The draw is an inverse CDF in token-id order.  A chunk is 512 consecutive
// ids, 8 per lane (one 16-byte load of bf16 logits); its sums are the lanes'
// sums reduced by a fixed butterfly, so every kernel that recomputes a chunk
// gets the same value.
// A residual draw compares p_t = e/Z (e = exp((x - m)/T)) with p_d token by
// token.  Rows without a nucleus carry a Z summed from float32 terms (within
// about 1e-6 of the fp64 sum), and the pass that computes the terms e is the
// one that would sum Z in fp64.  So the pass classifies each token with that
// Z: where p_t exceeds p_d by more than 1e-5 of p_d (then it does under the
// fp64 Z too) it adds e to a and p_d to b; it counts the tokens within that
// margin.  With Z = sum of e in fp64 (summed in the pick), the chunk's
// residual weight is a / Z - b; a chunk with a token inside the margin is
// summed again token by token with the fp64 Z.
// ---------------------------------------------------------------------------
constexpr int kDrawChunk = 512;       // ids per chunk: 8 per lane
constexpr int kDrawMaxChunks = 512;   // chunks of a row: 8 per lane of the pick scan
constexpr double kDrawMargin = 1e-5;  // relative margin of the row-pass Z's classification

// What the draw kernels need of a request, in one record.
struct Plan {
    int mode;     // kMode*
    int j;        // accepted drafts
    int row;      // row of the draw (residual or target modes)
    int fp64_z;   // residual draw of a row without a nucleus: Z summed again in fp64
    float m;      // the drawn row's maximum
    float lambda; // its nucleus threshold (-inf: every token)
    double zkeep; // its Z from the row statistics
    double invT;  // 1 / temperature
};

// Per-chunk sums of the draw pass (see above); b, a and unc only for
// residual draws.
struct ChunkRec {
    double a;  // sum of e over the tokens counted in the residual
    double b;  // sum of p_d over them
    double e;  // sum of e over the chunk
    int unc;   // tokens too close to p_t = p_d for the row-pass Z
    int pad;
};

// Logits (and, for residual draws, p_d) of the 8 consecutive tokens v0 ..
// v0+7 (-inf and 0 past the row end), with 16-byte loads when the rows are
// aligned.
template <typename T>
__device__ __forceinline__ void load8(const T* lr, const float* pd, int v0, int V, bool vec_ok,
                                      bool resid, float (&x)[8], float (&q)[8]) {
    if (vec_ok && v0 + 8 <= V) {
        if constexpr (sizeof(T) == 2) {
            const u32x4 lw = *(const u32x4*)(lr + v0);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = Logit<T>::lane(lw, e);
        } else {
            const u32x4 l0 = *(const u32x4*)(lr + v0), l1 = *(const u32x4*)(lr + v0 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = Logit<T>::lane(l0, e);
                x[e + 4] = Logit<T>::lane(l1, e);
            }
        }
        if (resid) {
            const f32x4 q0 = *(const f32x4*)(pd + v0), q1 = *(const f32x4*)(pd + v0 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                q[e] = q0[e];
                q[e + 4] = q1[e];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int v = v0 + e;
            x[e] = v < V ? Logit<T>::at(lr, v) : -INFINITY;
            q[e] = (resid && v < V) ? pd[v] : 0.f;
        }
    }
}

// Draw weights of the 8 consecutive tokens v0 .. v0+7 (0 past the row end):
// p = e * invZ, or the residual max(0, p - p_d).
template <typename T>
__device__ __forceinline__ void weights8(const T* lr, const float* pd, int v0, int V, bool vec_ok,
                                         bool resid, float lambda, float m, double invT,
                                         double invZ, const double* tab, double (&w)[8]) {
    float x[8], q[8];
    load8(lr, pd, v0, V, vec_ok, resid, x, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double p = (x[e] >= lambda) ? tempered(x[e], m, invT, tab) * invZ : 0.0;
        if (!resid) {
            w[e] = p;
        } else {
            const double r = p - (double)q[e];
            w[e] = r > 0.0 ? r : 0.0;
        }
    }
}

// The drawn row of a sampled request, as every draw block sees it.
template <typename T>
struct DrawRow {
    const T* lr;
    const float* pd;  // the draft's probabilities (residual draws)
    Plan pl;
    bool vec_ok;
    bool resid;       // residual max(0, p_t - p_d) rather than p_t

    __device__ DrawRow(const T* logits, const float* draft_probs, const Plan& p, int b, int K,
                       int V)
        : pl(p) {
        const int Q = K + 1;
        lr = logits + ((size_t)b * Q + pl.row) * V;
        resid = pl.mode == kModeResidual;
        pd = (resid && draft_probs) ? draft_probs + ((size_t)b * K + pl.row) * V : nullptr;
        vec_ok = (V % 8) == 0 && ((uintptr_t)lr & 15) == 0 &&
                 (pd == nullptr || ((uintptr_t)pd & 15) == 0);
    }
    // Lane `lane`'s 8 weights of chunk c and their sum (in id order).
    __device__ double lane_sum(int c, int lane, int V, bool res, double invZ, const double* tab,
                               double (&w)[8]) const {
        weights8(lr, pd, c * kDrawChunk + 8 * lane, V, vec_ok, res, pl.lambda, pl.m, pl.invT,
                 invZ, tab, w);
        double t = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) t += w[e];
        return t;
    }
    // Lane sums over its 8 ids of chunk c (see ChunkRec).
    __device__ void lane_rec(int c, int lane, int V, const double* tab, double& a, double& b,
                             double& e, int& unc) const {
        float x[8], q[8];
        load8(lr, pd, c * kDrawChunk + 8 * lane, V, vec_ok, resid, x, q);
        const double izc = 1.0 / pl.zkeep;
        const double margin = pl.fp64_z ? kDrawMargin : 0.0;
        a = b = e = 0.0;
        unc = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const double ev = (x[k] >= pl.lambda) ? tempered(x[k], pl.m, pl.invT, tab) : 0.0;
            e += ev;
            if (resid) {
                const double qd = (double)q[k];
                const double t = ev * izc - qd, tol = margin * fabs(qd);
                if (t > tol) {
                    a += ev;
                    b += qd;
                } else if (margin > 0.0 && t >= -tol && qd != 0.0) {
                    ++unc;
                }
            }
        }
    }
    // The ChunkRec of every chunk in [c_lo, c_hi), two in flight; f(c, rec)
    // gets each one (wave-uniform).
    template <typename F>
    __device__ void chunk_recs(int c_lo, int c_hi, int lane, int V, const double* tab,
                               F&& f) const {
        auto reduce = [&](double a, double b, double e, int unc) {
            ChunkRec r;
            r.e = wave_sum(e);
            if (resid) {
                r.a = wave_sum(a);
                r.b = wave_sum(b);
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) unc += shfl_xor(unc, m);
                r.unc = unc;
            } else {
                r.a = r.e;
                r.b = 0.0;
                r.unc = 0;
            }
            r.pad = 0;
            return r;
        };
        int c = c_lo;
        for (; c + 1 < c_hi; c += 2) {
            double a0, b0, e0, a1, b1, e1;
            int u0, u1;
            lane_rec(c, lane, V, tab, a0, b0, e0, u0);
            lane_rec(c + 1, lane, V, tab, a1, b1, e1, u1);
            f(c, reduce(a0, b0, e0, u0));
            f(c + 1, reduce(a1, b1, e1, u1));
        }
        if (c < c_hi) {
            double a0, b0, e0;
            int u0;
            lane_rec(c, lane, V, tab, a0, b0, e0, u0);
            f(c, reduce(a0, b0, e0, u0));
        }
    }
};

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v |= shfl_xor(v, m);
    return v;
}

// Lane n's value of v (every lane active).
__device__ __forceinline__ int lane_value(int v, int n) { return __shfl(v, n, 64); }

// The accept decision of request b, taken by one wave (every lane returns
// the same plan; loads are spread over the lanes, one per draft).  When
// `writer`, the wave also writes the request's outputs: all of them, except
// a sampled final token (next_token -1 and out_tokens[j] -1 until the draw
// fills them in).
__device__ Plan wave_plan(const int32_t* __restrict__ drafts, const float* __restrict__ temperature,
                          const float* __restrict__ draft_probs, const float* __restrict__ u_accept,
                          const int32_t* __restrict__ relaxed_topk, const float* __restrict__ top_p,
                          const RowStat* __restrict__ stats, int32_t* err, int b, int K, int V,
                          const int32_t* __restrict__ tree_parent, bool writer,
                          int32_t* __restrict__ num_accepted, int32_t* __restrict__ out_tokens,
                          int32_t* __restrict__ next_token, int32_t* __restrict__ accepted_nodes,
                          int lane) {
    const int Q = K + 1;
    int fl = 0;
    for (int r = lane; r < Q; r += 64) fl |= stats[(size_t)b * Q + r].flags;
    for (int n = lane; n < K; n += 64)
        if (drafts[(size_t)b * K + n] >= V) fl |= SD_DERR_TOKEN;
    const float Tb = temperature[b];
    // Trees (K + 1 <= 64 nodes, one per lane): node `lane`'s parent, draft
    // and row argmax.
    int par_l = -1, draft_l = -1, amax_l = -1;
    if (tree_parent && lane < Q) {
        par_l = tree_parent[(size_t)b * Q + lane];
        if (lane > 0) draft_l = drafts[(size_t)b * K + lane - 1];
    }
    fl = wave_or(fl);
    if (!fl && tree_parent) {
        // Strict greedy requests only, well-formed parents.
        const bool bad_l = lane < Q && (lane == 0 ? par_l != -1 : (par_l < 0 || par_l >= lane));
        if (Q > 64 || !(Tb == 0.f) || (relaxed_topk != nullptr && relaxed_topk[b] != 0) ||
            __ballot(bad_l) != 0)
            fl |= SD_DERR_TREE;
    }
    int mode = kModeInvalid, j = -1, row = 0, f = -1;
    unsigned long long path = 0;  // tree: bit n set for the kept path's nodes
    int depth_l = 0;              // tree: depth of node `lane`
    if (fl) {
        if (writer && lane == 0) set_error(err, fl);
    } else if (tree_parent) {
        // Node n is accepted when its parent is (the root always is) and its
        // draft is the parent row's argmax.  One pass in node order (parents
        // first, every lane the same) gives every node's depth and
        // acceptance; the deepest accepted node, the first one found on ties
        // (smallest index), ends the kept path.
        if (lane < Q) amax_l = stats[(size_t)b * Q + lane].argmax;
        unsigned long long acc = 1;  // bit n: node n accepted
        int best = 0, best_depth = 0;
        for (int n = 1; n < Q; ++n) {
            const int p = lane_value(par_l, n), d = lane_value(draft_l, n);
            const int dn = lane_value(depth_l, p) + 1;
            if (lane == n) depth_l = dn;
            if (((acc >> p) & 1) && d >= 0 && d == lane_value(amax_l, p)) {
                acc |= 1ull << n;
                if (dn > best_depth) {
                    best = n;
                    best_depth = dn;
                }
            }
        }
        for (int c = best; c != 0; c = lane_value(par_l, c)) path |= 1ull << c;
        j = best_depth;
        f = lane_value(amax_l, best);
        mode = kModeTree;
    } else if (Tb == 0.f) {
        // Strict: the draft must be the row's argmax.  Relaxed (top-N > 0):
        // it must survive the row's top-N / delta filter.  j = the first
        // draft that fails.
        const bool relaxed = relaxed_topk != nullptr && relaxed_topk[b] > 0;
        j = K;
        for (int base = 0; base < K; base += 64) {
            const int n = base + lane;
            bool fail = false;
            if (n < K) {
                const int d = drafts[(size_t)b * K + n];
                const RowStat& st = stats[(size_t)b * Q + n];
                fail = d < 0 || !(relaxed ? st.relaxed_ok != 0 : d == st.argmax);
            }
            const unsigned long long m = __ballot(fail);
            if (m) {
                j = base + __ffsll((long long)m) - 1;
                break;
            }
        }
        f = stats[(size_t)b * Q + j].argmax;
        mode = kModeDone;
    } else {
        // Rejection sampling: draft n+1 is kept while u < min(1, p_t/p_d);
        // the first rejection draws from the residual of its row, a full
        // chain (or a missing draft) from p_t of the next row.
        j = K;
        row = K;
        mode = kModeTarget;
        for (int base = 0; base < K; base += 64) {
            const int n = base + lane;
            int kind = 0;  // 0 kept, 1 missing draft, 2 rejected
            if (n < K) {
                const int d = drafts[(size_t)b * K + n];
                if (d < 0) {
                    kind = 1;
                } else {
                    const double a = stats[(size_t)b * Q + n].pt_d;
                    const double qd = draft_probs[((size_t)b * K + n) * V + d];
                    const double ratio = qd > 0.0 ? a / qd : (a > 0.0 ? INFINITY : 0.0);
                    const double accp = ratio < 1.0 ? ratio : 1.0;
                    if (!((double)u_accept[(size_t)b * Q + n] < accp)) kind = 2;
                }
            }
            const unsigned long long m = __ballot(kind != 0);
            if (m) {
                const int first = __ffsll((long long)m) - 1;
                j = row = base + first;
                mode = lane_value(kind, first) == 2 ? kModeResidual : kModeTarget;
                break;
            }
        }
    }
    if (writer) {
        if (lane == 0) {
            num_accepted[b] = j;
            next_token[b] = f;  // -1 for invalid requests and sampled tokens
        }
        for (int k = lane; k < Q; k += 64) {
            int tok = -1;
            if (mode != kModeInvalid && mode != kModeTree && k < j) tok = drafts[(size_t)b * K + k];
            else if (mode != kModeInvalid && k == j) tok = f;
            if (!(mode == kModeTree && k < j)) out_tokens[(size_t)b * Q + k] = tok;
            if (accepted_nodes && !(mode == kModeTree && k >= 1 && k <= j))
                accepted_nodes[(size_t)b * Q + k] =
                    mode == kModeInvalid ? -1 : (k == 0 ? 0 : (k <= j ? k : -1));
        }
        if (mode == kModeTree && lane < Q && ((path >> lane) & 1)) {
            // The kept path's nodes, each at its depth.
            if (accepted_nodes) accepted_nodes[(size_t)b * Q + depth_l] = lane;
            out_tokens[(size_t)b * Q + depth_l - 1] = draft_l;
        }
    }
    Plan pl;
    pl.mode = mode;
    pl.j = j;
    pl.row = row;
    pl.fp64_z = 0;
    pl.m = 0.f;
    pl.lambda = -INFINITY;
    pl.zkeep = 1.0;
    pl.invT = 1.0;
    if (mode == kModeResidual || mode == kModeTarget) {
        const RowStat st = stats[(size_t)b * Q + row];
        pl.m = st.m;
        pl.lambda = st.lambda;
        pl.zkeep = st.zkeep;
        pl.invT = 1.0 / (double)Tb;
        // The row pass summed Z of a row without a nucleus from float32
        // terms.  A draw from p_t is indifferent to a common scale, but the
        // residual compares p_t with p_d token by token, so its Z is summed
        // again in fp64.  A nucleus row's kept mass is fp64 already.
        pl.fp64_z = mode == kModeResidual && (top_p == nullptr || !(top_p[b] < 1.f));
    }
    return pl;
}

// One wave per request, four per block.
__global__ __launch_bounds__(256) void accept_plan(
    const int32_t* __restrict__ drafts, const float* __restrict__ temperature,
    const float* __restrict__ draft_probs, const float* __restrict__ u_accept,
    const float* __restrict__ top_p, const int32_t* __restrict__ relaxed_topk,
    const RowStat* __restrict__ stats, Plan* __restrict__ plans,
    int32_t* __restrict__ num_accepted, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ next_token, int32_t* err, int B, int K, int V,
    const int32_t* __restrict__ tree_parent, int32_t* __restrict__ accepted_nodes) {
    const int lane = threadIdx.x & 63, b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= B) return;
    const Plan pl = wave_plan(drafts, temperature, draft_probs, u_accept, relaxed_topk, top_p,
                              stats, err, b, K, V, tree_parent, true, num_accepted, out_tokens,
                              next_token, accepted_nodes, lane);
    if (lane == 0) plans[b] = pl;
}

// Grid: batch x ns blocks of 256 threads; slice s covers chunks
// [4 cpw s, 4 cpw (s + 1)), cpw per wave.
template <typename T>
__global__ __launch_bounds__(256) void accept_draw_w(const T* __restrict__ logits,
                                                     const float* __restrict__ draft_probs,
                                                     const Plan* __restrict__ plans,
                                                     ChunkRec* __restrict__ recs, int K, int V,
                                                     int ns, int cpw) {
    const int b = blockIdx.x / ns, s = blockIdx.x - b * ns;
    const Plan pl = plans[b];
    if (pl.mode != kModeResidual && pl.mode != kModeTarget) return;
    const DrawRow<T> dr(logits, draft_probs, pl, b, K, V);
    __shared__ double s_exptab[64];
    exp_table_init(s_exptab);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nchunks = (V + kDrawChunk - 1) / kDrawChunk;
    ChunkRec* rc = recs + (size_t)b * nchunks;
    const int c_lo = min(nchunks, (4 * s + wave) * cpw), c_hi = min(nchunks, c_lo + cpw);
    dr.chunk_recs(c_lo, c_hi, lane, V, s_exptab, [&](int c, const ChunkRec& r) {
        if (lane == 0) rc[c] = r;
    });
}

// Wave 0 of the pick: lane l owns chunks [l cpl, (l+1) cpl); their sums are
// added in chunk order per lane, then scanned across lanes in lane order.
// Returns the row total; *pre = the lane's exclusive prefix, *own its sum.
__device__ __forceinline__ double scan_chunks(const double* cs, int nchunks, int cpl, int lane,
                                              double* pre, double* own) {
    double t = 0.0;
    const int c_lo = lane * cpl, c_hi = min(nchunks, c_lo + cpl);
    for (int c = c_lo; c < c_hi; ++c) t += cs[c];
    double incl = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    *pre = incl - t;
    *own = t;
    return __shfl(incl, 63, 64);
}

// One block per request.
template <typename T>
__global__ __launch_bounds__(256) void accept_draw_pick(
    const T* __restrict__ logits, const float* __restrict__ draft_probs,
    const float* __restrict__ u_sample, const Plan* __restrict__ plans,
    const ChunkRec* __restrict__ recs, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ next_token, int K, int V) {
    const int b = blockIdx.x;
    const Plan pl = plans[b];
    if (pl.mode != kModeResidual && pl.mode != kModeTarget) return;
    const DrawRow<T> dr(logits, draft_probs, pl, b, K, V);
    __shared__ double s_exptab[64];
    __shared__ double s_cs[kDrawMaxChunks], s_e[kDrawMaxChunks], s_b[kDrawMaxChunks];
    __shared__ int s_unc[kDrawMaxChunks];
    __shared__ double s_total, s_pre, s_invz;
    __shared__ int s_chunk, s_f;
    __shared__ int s_cand[4];
    exp_table_init(s_exptab);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Q = K + 1;
    const int nchunks = (V + kDrawChunk - 1) / kDrawChunk;
    const int cpl = (nchunks + 63) / 64;
    const ChunkRec* rc = recs + (size_t)b * nchunks;
    const double u = (double)u_sample[(size_t)b * Q + pl.row];
    for (int c = tid; c < nchunks; c += 256) {
        const ChunkRec r = rc[c];
        s_e[c] = r.e;
        s_cs[c] = r.a;  // (the residual's weight sum is formed below)
        s_b[c] = r.b;
        s_unc[c] = r.unc;
    }
    __syncthreads();
    bool resid = dr.resid;
    double invZ = 1.0;  // p_t unnormalised (the draw is scale-free), unless residual
    if (resid) {
        if (wave == 0) {
            double z = 1.0 / pl.zkeep;
            if (pl.fp64_z) {  // Z = the fp64 terms of every chunk, in a fixed order
                double pre, own;
                z = 1.0 / scan_chunks(s_e, nchunks, cpl, lane, &pre, &own);
            }
            if (lane == 0) s_invz = z;
        }
        __syncthreads();
        invZ = s_invz;
        for (int c = tid; c < nchunks; c += 256) s_cs[c] = fmax(s_cs[c] * invZ - s_b[c], 0.0);
        __syncthreads();
        if (pl.fp64_z) {
            // Chunks with a token inside the margin: summed again token by
            // token with the fp64 Z.
            for (int c = wave; c < nchunks; c += 4) {
                if (s_unc[c] == 0) continue;
                double w[8];
                const double t = wave_sum(dr.lane_sum(c, lane, V, true, invZ, s_exptab, w));
                if (lane == 0) s_cs[c] = t;
            }
            __syncthreads();
        }
    }
    if (wave == 0) {
        double pre, own;
        const double tot = scan_chunks(s_cs, nchunks, cpl, lane, &pre, &own);
        if (lane == 0) s_total = tot;
    }
    __syncthreads();
    if (resid && s_total == 0.0) {
        // The residual is empty: the draw takes p_t itself (unnormalised).
        for (int c = tid; c < nchunks; c += 256) s_cs[c] = s_e[c];
        resid = false;
        invZ = 1.0;
        __syncthreads();
    }
    if (wave == 0) {
        // The crossing lane: the first whose running sum exceeds u * total.
        // It walks its chunks, added one by one (another order than its lane
        // sum), so rounding may leave every chunk short of the target: then
        // its last chunk of positive weight is taken (the search inside the
        // chunk then ends on its last positive token).
        double pre, own;
        const double tot = scan_chunks(s_cs, nchunks, cpl, lane, &pre, &own);
        const double target = u * tot;
        const unsigned long long cross = __ballot(pre + own > target);
        int fc = -1;
        double run_at = 0.0;
        if (cross) {
            const int cl = __ffsll((long long)cross) - 1;
            if (lane == cl) {
                const int c_lo = lane * cpl, c_hi = min(nchunks, c_lo + cpl);
                double run = pre, pre_last = pre;
                int lastpos = -1;
                for (int c = c_lo; c < c_hi; ++c) {
                    const double v = s_cs[c];
                    if (run + v > target) {
                        fc = c;
                        break;
                    }
                    if (v > 0.0) {
                        lastpos = c;
                        pre_last = run;
                    }
                    run += v;
                }
                if (fc < 0) {
                    fc = lastpos;
                    run = pre_last;
                }
                run_at = run;
            }
            fc = __shfl(fc, cl, 64);
            run_at = __shfl(run_at, cl, 64);
        }
        if (lane == 0) {
            s_chunk = fc;
            s_pre = run_at;
            s_total = tot;
        }
    }
    __syncthreads();
    if (s_chunk >= 0 && wave == 0) {
        // Inside the chunk: lane-order inclusive scan of the lanes' sums,
        // then the crossing lane walks its 8 tokens in order.  If rounding
        // leaves the target beyond the chunk, take its last positive token.
        const int c = s_chunk;
        double w[8];
        const double t = dr.lane_sum(c, lane, V, resid, invZ, s_exptab, w);
        double incl = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const double target = u * s_total;
        const unsigned long long mask = __ballot(s_pre + incl > target);
        if (mask) {
            const int hl = __ffsll((long long)mask) - 1;
            if (lane == hl) {
                double run = s_pre + incl - t;
                int pick = -1, lastpos = -1;
                for (int e = 0; e < 8; ++e) {
                    if (w[e] > 0.0) lastpos = e;
                    run += w[e];
                    if (run > target && pick < 0) pick = e;
                }
                if (pick < 0) pick = lastpos;
                s_f = c * kDrawChunk + 8 * lane + pick;
            }
        } else {
            int lp = -1;
            for (int e = 0; e < 8; ++e)
                if (w[e] > 0.0) lp = e;
            const unsigned long long pm = __ballot(lp >= 0);
            const int top = pm ? 63 - __clzll((long long)pm) : -1;
            if (lane == 0) s_f = -1;
            if (top >= 0 && lane == top) s_f = c * kDrawChunk + 8 * lane + lp;
        }
    } else if (tid == 0) {
        s_f = -1;
    }
    __syncthreads();
    if (s_f < 0) {
        // Rounding left no bucket above the target: the largest id with
        // positive weight.
        int cand = -1;
        for (int c = nchunks - 1 - wave; c >= 0 && cand < 0; c -= 4) {
            double w[8];
            dr.lane_sum(c, lane, V, resid, invZ, s_exptab, w);
            int lp = -1;
            for (int e = 0; e < 8; ++e)
                if (w[e] > 0.0) lp = e;
            const unsigned long long pm = __ballot(lp >= 0);
            if (pm) {
                const int top = 63 - __clzll((long long)pm);
                const int lpt = __shfl(lp, top, 64);
                cand = c * kDrawChunk + 8 * top + lpt;
            }
        }
        if (lane == 0) s_cand[wave] = cand;
        __syncthreads();
        if (tid == 0) {
            int f = -1;
            for (int w = 0; w < 4; ++w) f = max(f, s_cand[w]);
            s_f = f;
        }
        __syncthreads();
    }
    if (tid == 0) {
        next_token[b] = s_f;
        out_tokens[(size_t)b * Q + pl.j] = s_f;
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

// Slices per row for the row statistics: slices of at least 2048 ids, at
// most 32 per row.  span is a multiple of 8 ids so every slice starts on a
// 16-byte vector.
void row_split(int rows, int V, int* splits, int* span) {
    // About 1024 blocks in all (measured: 1152 blocks of 5336 ids beat 2112
    // of 2912 at 192 x 32000, 1024 beat 2048 at 256 x 129280), but at least
    // two slices per row of a long vocabulary (2560 blocks beat 1280 at
    // 1280 x 129280).
    int sp = (1024 + rows - 1) / rows;
    if (V >= 65536) sp = std::max(sp, 2);
    sp = std::min(sp, std::max(1, V / 2048));
    sp = std::max(1, std::min(sp, 32));
    int sn = (V + sp - 1) / sp;
    sn = (sn + 7) & ~7;
    *span = sn;
    *splits = (V + sn - 1) / sn;
}

// Chunks per wave of the draw pass (two loads in flight per lane; more per
// wave measured slower).
int draw_cpw(int, int) { return 2; }

// Slices (blocks) per row of the draw passes.
int draw_slices(int B, int V) {
    const int nchunks = (V + kDrawChunk - 1) / kDrawChunk;
    const int per_block = 4 * draw_cpw(B, V);
    return (nchunks + per_block - 1) / per_block;
}

// Workspace: row statistics, slice records, then the draw's plans, Z slice
// sums and chunk sums, each 256-byte aligned.
struct AcceptWs {
    size_t stats, parts, plans, recs, total;
};

AcceptWs accept_ws_layout(const sd_accept_desc* d) {
    const int rows = d->batch * (d->K + 1);
    int splits, span;
    row_split(rows, d->vocab, &splits, &span);
    const size_t B = (size_t)d->batch;
    const size_t nchunks = (size_t)(d->vocab + kDrawChunk - 1) / kDrawChunk;
    AcceptWs w;
    w.stats = 0;
    w.parts = w.stats + align_up(sizeof(RowStat) * (size_t)rows, 256);
    w.plans = w.parts + align_up(sizeof(RowPart) * (size_t)rows * splits, 256);
    w.recs = w.plans + align_up(sizeof(Plan) * B, 256);
    w.total = w.recs + align_up(sizeof(ChunkRec) * B * nchunks, 256);
    return w;
}

size_t accept_ws_bytes(const sd_accept_desc* d) { return accept_ws_layout(d).total; }

int check_accept(const sd_accept_desc* d) {
    if (!d) return fail(SD_EINVAL, "sd_accept_desc is NULL");
    if (d->batch <= 0 || d->K < 0 || d->vocab <= 0)
        return fail(SD_EINVAL, "sd_accept: bad batch/K/vocab");
    if (d->logits_dtype != SD_BF16 && d->logits_dtype != SD_F32)
        return fail(SD_EINVAL, "sd_accept: unknown logits dtype %d", d->logits_dtype);
    if ((long)d->batch * (d->K + 1) > 0x7fffffffL)
        return fail(SD_EUNSUPPORTED, "sd_accept: too many rows");
    if ((long)d->vocab > (long)kDrawMaxChunks * kDrawChunk)
        return fail(SD_EUNSUPPORTED, "sd_accept: vocab above %d", kDrawMaxChunks * kDrawChunk);
    if ((long)d->batch * draw_slices(d->batch, d->vocab) > 0x7fffffffL)
        return fail(SD_EUNSUPPORTED, "sd_accept: too many draw blocks");
    if (d->tree_parent && d->K + 1 > 64)
        return fail(SD_EUNSUPPORTED, "sd_accept: a draft tree needs K+1 <= 64, got %d", d->K + 1);
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

namespace sdv {
namespace {

int check_accept_pointers(const sd_accept_desc* d, const char* what) {
    if (!d->logits || !d->temperature || !d->u_accept || !d->u_sample || !d->num_accepted ||
        !d->out_tokens || !d->next_token || !d->out_offsets || !d->packed_tokens ||
        (d->K > 0 && !d->draft_tokens))
        return fail(SD_EINVAL, "%s: NULL required pointer", what);
    return SD_OK;
}

// The decision and the draw.  A sampled request with drafts needs
// draft_probs (otherwise the row merge marks it invalid), so without them
// and K > 0 no request draws and the draw kernels are skipped.
template <typename T>
int draw_launch(const T* lg, const sd_accept_desc* d, const RowStat* stats, Plan* plans,
                ChunkRec* recs, hipStream_t s) {
    int rc;
    const int B = d->batch, K = d->K, V = d->vocab;
    accept_plan<<<(B + 3) / 4, 256, 0, s>>>(d->draft_tokens, d->temperature, d->draft_probs,
                                            d->u_accept, d->top_p, d->relaxed_topk, stats, plans,
                                            d->num_accepted, d->out_tokens, d->next_token,
                                            d->dev_error, B, K, V, d->tree_parent,
                                            d->accepted_nodes);
    if ((rc = check_launch("accept_plan")) != SD_OK) return rc;
    if (d->draft_probs == nullptr && K > 0) return SD_OK;
    const int ns = draw_slices(B, V), cpw = draw_cpw(B, V);
    const unsigned grid = (unsigned)((long)B * ns);
    accept_draw_w<T><<<grid, 256, 0, s>>>(lg, d->draft_probs, plans, recs, K, V, ns, cpw);
    if ((rc = check_launch("accept_draw_w")) != SD_OK) return rc;
    accept_draw_pick<T><<<B, 256, 0, s>>>(lg, d->draft_probs, d->u_sample, plans, recs,
                                          d->out_tokens, d->next_token, K, V);
    return check_launch("accept_draw_pick");
}

// The kernels of one acceptance call, with the row statistics and slice
// records in `workspace` (accept_ws_bytes(d) bytes, 256-byte aligned; no
// initialisation needed: every record is written before it is read).
int accept_launch(const sd_accept_desc* d, void* workspace, hipStream_t s) {
    int rc;
    const int B = d->batch, K = d->K, V = d->vocab, Q = K + 1;
    const int rows = B * Q;
    int splits, span;
    row_split(rows, V, &splits, &span);
    const AcceptWs ws = accept_ws_layout(d);
    char* w0 = (char*)workspace;
    RowStat* stats = (RowStat*)(w0 + ws.stats);
    RowPart* parts = (RowPart*)(w0 + ws.parts);
    Plan* plans = (Plan*)(w0 + ws.plans);
    ChunkRec* recs = (ChunkRec*)(w0 + ws.recs);
    const int es = d->logits_dtype == SD_BF16 ? 2 : 4;
    const int vec_ok = aligned16(d->logits) && ((size_t)V * es) % 16 == 0;
    const int has_probs = d->draft_probs != nullptr;
    if (d->logits_dtype == SD_BF16) {
        const uint16_t* lg = (const uint16_t*)d->logits;
        if (d->relaxed_topk)
            accept_rowpart<uint16_t, true><<<rows * splits, 256, 0, s>>>(
                lg, d->draft_tokens, d->temperature, d->top_p, d->relaxed_topk, parts, Q, V, splits,
                span, vec_ok);
        else
            accept_rowpart<uint16_t, false><<<rows * splits, 256, 0, s>>>(
                lg, d->draft_tokens, d->temperature, d->top_p, nullptr, parts, Q, V, splits, span,
                vec_ok);
        if ((rc = check_launch("accept_rowpart")) != SD_OK) return rc;
        accept_rowmerge<uint16_t><<<(rows + 3) / 4, 256, 0, s>>>(
            lg, d->draft_tokens, d->temperature, d->top_p, has_probs, d->relaxed_topk,
            d->relaxed_delta, parts, stats, rows, K, V, splits);
        if ((rc = check_launch("accept_rowmerge")) != SD_OK) return rc;
        if (d->top_p) {
            accept_topp_bf16<<<rows, kToppThreads, kWin * sizeof(uint32_t), s>>>(
                lg, d->draft_tokens, d->temperature, d->top_p, stats, K, V, vec_ok);
            if ((rc = check_launch("accept_topp_bf16")) != SD_OK) return rc;
        }
        if ((rc = draw_launch(lg, d, stats, plans, recs, s)) != SD_OK) return rc;
    } else {
        const float* lg = (const float*)d->logits;
        if (d->relaxed_topk)
            accept_rowpart<float, true><<<rows * splits, 256, 0, s>>>(
                lg, d->draft_tokens, d->temperature, d->top_p, d->relaxed_topk, parts, Q, V, splits,
                span, vec_ok);
        else
            accept_rowpart<float, false><<<rows * splits, 256, 0, s>>>(
                lg, d->draft_tokens, d->temperature, d->top_p, nullptr, parts, Q, V, splits, span,
                vec_ok);
        if ((rc = check_launch("accept_rowpart")) != SD_OK) return rc;
        accept_rowmerge<float><<<(rows + 3) / 4, 256, 0, s>>>(
            lg, d->draft_tokens, d->temperature, d->top_p, has_probs, d->relaxed_topk,
            d->relaxed_delta, parts, stats, rows, K, V, splits);
        if ((rc = check_launch("accept_rowmerge")) != SD_OK) return rc;
        if (d->top_p) {
            accept_topp_f32<<<rows, 256, 0, s>>>(lg, d->draft_tokens, d->temperature, d->top_p,
                                                 stats, K, V, vec_ok);
            if ((rc = check_launch("accept_topp_f32")) != SD_OK) return rc;
        }
        if ((rc = draw_launch(lg, d, stats, plans, recs, s)) != SD_OK) return rc;
    }
    accept_pack<<<1, 1024, 0, s>>>(d->num_accepted, d->out_tokens, d->out_offsets,
                                   d->packed_tokens, B, Q);
    return check_launch("accept_pack");
}

// ---------------------------------------------------------------------------
// Scratch of sd_accept_noalloc: a fixed device array instead of a caller
// workspace, for callers that cannot allocate.  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never names the
// array in a launch or a copy: its name there is a host-side stand-in, so
// the device address is looked up once per device with hipGetSymbolAddress
// and kept in g_scratch_ptr.
// ---------------------------------------------------------------------------
constexpr size_t kAcceptScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device, with the device current).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(SD_EDEVICE, "sd_accept_noalloc: no usable current device");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(SD_EDEVICE, "sd_accept_noalloc: scratch address on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SD_OK;
}

}  // namespace
}  // namespace sdv

extern "C" int sd_accept(const sd_accept_desc* d, void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    int rc = check_accept(d);
    if (rc != SD_OK) return rc;
    if ((rc = check_accept_pointers(d, "sd_accept")) != SD_OK) return rc;
    if (!workspace || !aligned256(workspace))
        return fail(SD_EINVAL, "sd_accept: workspace NULL or not 256-byte aligned");
    const size_t need = accept_ws_bytes(d);
    if (ws_bytes < need) return fail(SD_EWORKSPACE, "sd_accept: workspace %zu < %zu", ws_bytes, need);
    return accept_launch(d, workspace, (hipStream_t)stream);
}

extern "C" int sd_accept_noalloc(const sd_accept_desc* d, void* stream) {
    clear_error();
    int rc = check_accept(d);
    if (rc != SD_OK) return rc;
    if ((rc = check_accept_pointers(d, "sd_accept_noalloc")) != SD_OK) return rc;
    const size_t need = accept_ws_bytes(d);
    if (need > kAcceptScratchBytes)
        return fail(SD_EWORKSPACE,
                    "sd_accept_noalloc: this batch needs %zu bytes of scratch, above the fixed "
                    "%zu (use sd_accept with a workspace)", need, kAcceptScratchBytes);
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != SD_OK) return rc;
    return accept_launch(d, ws, (hipStream_t)stream);
}
