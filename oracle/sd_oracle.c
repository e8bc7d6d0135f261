/*
 * sd_oracle.c -- TEST INFRASTRUCTURE.  The slow, plain, fp64 CPU oracle of
 * the speculative-decoding verify step.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it; the product library
 * never does.  It shares no code, header, table or helper with the HIP
 * path.  Every function is a direct loop nest over the definition it
 * cites, accumulating in double precision, with no blocking or fusion.
 * OpenMP splits only the outermost independent loop (one output row or
 * one output element per iteration), which leaves every sum's order fixed.
 *
 * Pages cited (titles and sections; the text is Chinese):
 *   [TRT-MTP]     TensorRT-LLM MTP implementation/optimisation article
 *                 (makelele.cn/d/6983435): "背景" with Fig. 1 (verify
 *                 example), "MTP Vanilla"/"MTP Eagle" (clearing rejected
 *                 KV), "基本實現方式" with Fig. 4 (rollback outside the
 *                 engine), "支持 MTP 的注意力機制" (causal mask over K+1
 *                 queries), "寬松接受" (relaxed acceptance).
 *   [SD-PRACTICE] "推测解码与MTP：大模型推理加速的核心技术与工程实践"
 *                 (mlqm.cn/news/1017475): s2.2 parallel verify, s2.3
 *                 accept/correct, s4.3 KV cache, s4.4 sampling rules.
 *   [CSDN-MTP]    CSDN article on the two meanings of "MTP"
 *                 (gitcode.csdn.net/69b64a3354b52172bc617fab): "整体计算流程
 *                 （以 K=3 草稿 Token 为例）" steps 2 (attention formula and
 *                 table), 4 (output layer), 5 (softmax), 6 (compare);
 *                 "回滚机制仅修正错误，不重复计算" (rollback).
 *   [VLLM-MTP]    "MPT (MTP, Multi-Token Prediction) 原理详解"
 *                 (mqxn.cn/news/75683): s3 stages 3-4 (greedy and
 *                 rejection-sampling verify, 1..D+1 outputs), s4 worked
 *                 example and counter-example, s5 losslessness.
 *
 * Readings taken where the pages are silent or disagree (each is also a test):
 *   - draft n is judged by logits row n-1 (row i predicts position i+1);
 *   - query i attends to keys 0 .. L_b+i, its own key included;
 *   - acceptance is u < min(1, p_t/p_d) with u in [0,1);
 *   - the replacement token is drawn from norm(max(0, p_t - p_d)); with a
 *     one-hot p_d this is p_t with the draft removed;
 *   - argmax ties go to the smallest token id;
 *   - top-p keeps the shortest prefix of (logit desc, id asc) whose tempered
 *     mass reaches top_p, extended to every token tied with its last logit;
 *   - an FP8 KV cache holds OCP E4M3 ("fn") codes with one key scale and one
 *     value scale per kv head; appending stores the nearest code (ties to
 *     even, saturating at 448, NaN kept) of value / scale;
 *   - a tree of drafts lists its nodes in topological order (root 0,
 *     parent[i] < i); a node attends to its ancestors and itself; greedy
 *     verification keeps the longest accepted root-to-node path (a node is
 *     accepted when its parent is and its draft is the parent row's argmax;
 *     the smallest end-node index among equally long paths); the accepted
 *     path's rows are gathered to contiguous slots.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2, ORC_E4M3 = 3 };
enum { ORC_OK = 0, ORC_EARG = 1, ORC_EPAGE = 2 };

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------
 * FP8 cache codes: the OCP 8-bit floating-point format E4M3 in its "fn"
 * variant (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; 0x7F and 0xFF are NaN, so the largest finite value is
 * 1.75 * 2^8 = 448; exponent field 0 holds the subnormals m/8 * 2^-6).
 * The pages name FP8 attention only as prior art ([TRT-MTP] "支持 MTP 的注意力
 * 機制": FP8 FlashMLA); the cache format is this reading of it.  A cached
 * element stands for code_value * scale[kv head], with one scale for keys
 * and one for values per kv head.
 * ---------------------------------------------------------------------- */
double orc_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Code of x: NaN -> 0x7F; otherwise the sign bit of x and the code of the
 * representable magnitude nearest to min(|x|, 448) (saturation), ties to the
 * code with an even mantissa, found by trying every finite magnitude code
 * 0x00 .. 0x7E (their values increase with the code). */
uint8_t orc_e4m3_code(double x) {
    if (isnan(x)) return 0x7F;
    double a = fabs(x);
    if (a > 448.0) a = 448.0;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(orc_e4m3_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)((signbit(x) ? 0x80 : 0) | best);
}

void orc_e4m3_decode(const uint8_t* codes, double* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_e4m3_value(codes[i]);
}

void orc_e4m3_encode(const double* x, uint8_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_e4m3_code(x[i]);
}

/* Element i of an array stored as float32, bfloat16 bits, float64, or E4M3
 * codes (the code's value; a cache scale is applied by the caller). */
static double load_elem(const void* p, int dtype, size_t i) {
    if (dtype == ORC_F32) return (double)((const float*)p)[i];
    if (dtype == ORC_F64) return ((const double*)p)[i];
    if (dtype == ORC_E4M3) return orc_e4m3_value(((const uint8_t*)p)[i]);
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t elem_size(int dtype) {
    return dtype == ORC_F32 ? 4 : dtype == ORC_F64 ? 8 : dtype == ORC_E4M3 ? 1 : 2;
}

/* ------------------------------------------------------------------------
 * Rounding of exact values to the stored output types.
 * bf16: round-to-nearest, ties to even, straight from the double (one
 * rounding).  The spacing of bf16 numbers in [2^e, 2^(e+1)) is 2^(e-7);
 * below 2^-126 it is the subnormal spacing 2^-133.
 * ---------------------------------------------------------------------- */
void orc_round_bf16(const double* x, uint16_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) {
        double v = x[i];
        float f;
        if (isnan(v)) {
            f = NAN;
        } else if (v == 0.0 || isinf(v)) {
            f = (float)v;
        } else {
            int e;
            frexp(fabs(v), &e);          /* |v| = m * 2^e, m in [0.5, 1) */
            int ex = e - 1;              /* |v| in [2^ex, 2^(ex+1)) */
            if (ex < -126) ex = -126;
            double ulp = ldexp(1.0, ex - 7);
            double r = nearbyint(v / ulp) * ulp;   /* ties to even */
            if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, v);
            f = (float)r;                /* exact: r is a bf16 value */
        }
        uint32_t bits;
        memcpy(&bits, &f, sizeof bits);
        out[i] = (uint16_t)(bits >> 16);
    }
}

void orc_round_f32(const double* x, float* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = (float)x[i];
}

/* ------------------------------------------------------------------------
 * Paged KV cache addressing.  Position p of request b lives in logical page
 * p / page_size at offset p % page_size; the page table maps the logical
 * page to a physical page of the pool.
 * GQA cache: [num_pages][n_kv_heads][page_size][d].
 * MLA cache (one latent vector per position): [num_pages][page_size][d].
 * ---------------------------------------------------------------------- */
static long phys_page(const int* page_table, int max_pages, int num_pages, int b,
                      long pos, int page_size) {
    long lp = pos / page_size;
    if (lp < 0 || lp >= max_pages) return -1;
    long pg = page_table[(size_t)b * max_pages + lp];
    if (pg < 0 || pg >= num_pages) return -1;
    return pg;
}

static size_t gqa_index(long page, int h, int n_kv_heads, int page_size, long off,
                        int d, int dd) {
    return (((size_t)page * n_kv_heads + h) * page_size + off) * d + dd;
}

/*
 * Append: the K+1 new keys/values of request b go to positions
 * L_b .. L_b+K of its cache, so that later queries of the same step can
 * read them ([CSDN-MTP] step 2: each new K/V is written into the cache as
 * soon as it is produced).  For MLA, k_new is the latent vector and v_new
 * is unused.  The cache arrays and the new rows share one dtype.
 */
int orc_kv_append(int B, int Q, int n_kv_heads, int d_k, int d_v, int mla, int page_size,
                  int max_pages, int num_pages, int dtype, const void* k_new,
                  const void* v_new, void* k_cache, void* v_cache, const int* page_table,
                  const int* seq_lens) {
    size_t es = elem_size(dtype);
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < Q; ++i) {
            long pos = (long)seq_lens[b] + i;
            long pg = phys_page(page_table, max_pages, num_pages, b, pos, page_size);
            if (pg < 0) return ORC_EPAGE;
            long off = pos % page_size;
            if (mla) {
                for (int d = 0; d < d_k; ++d) {
                    size_t dst = ((size_t)pg * page_size + off) * d_k + d;
                    size_t src = ((size_t)b * Q + i) * d_k + d;
                    memcpy((char*)k_cache + dst * es, (const char*)k_new + src * es, es);
                }
                continue;
            }
            for (int h = 0; h < n_kv_heads; ++h) {
                for (int d = 0; d < d_k; ++d) {
                    size_t dst = gqa_index(pg, h, n_kv_heads, page_size, off, d_k, d);
                    size_t src = (((size_t)b * Q + i) * n_kv_heads + h) * d_k + d;
                    memcpy((char*)k_cache + dst * es, (const char*)k_new + src * es, es);
                }
                for (int d = 0; d < d_v; ++d) {
                    size_t dst = gqa_index(pg, h, n_kv_heads, page_size, off, d_v, d);
                    size_t src = (((size_t)b * Q + i) * n_kv_heads + h) * d_v + d;
                    memcpy((char*)v_cache + dst * es, (const char*)v_new + src * es, es);
                }
            }
        }
    }
    return ORC_OK;
}

/*
 * Append into an FP8 (E4M3) cache: as orc_kv_append, but element d of new
 * row (b, i, h) is stored as the code of value / scale[h] (k_scale for keys,
 * v_scale for values), so that code_value * scale is the nearest the cache
 * can hold to the new value.  new_dtype is the type of k_new/v_new.
 */
int orc_kv_append_e4m3(int B, int Q, int n_kv_heads, int d_k, int d_v, int page_size,
                       int max_pages, int num_pages, int new_dtype, const void* k_new,
                       const void* v_new, uint8_t* k_cache, uint8_t* v_cache,
                       const int* page_table, const int* seq_lens, const float* k_scale,
                       const float* v_scale) {
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < Q; ++i) {
            long pos = (long)seq_lens[b] + i;
            long pg = phys_page(page_table, max_pages, num_pages, b, pos, page_size);
            if (pg < 0) return ORC_EPAGE;
            long off = pos % page_size;
            for (int h = 0; h < n_kv_heads; ++h) {
                for (int d = 0; d < d_k; ++d) {
                    size_t src = (((size_t)b * Q + i) * n_kv_heads + h) * d_k + d;
                    k_cache[gqa_index(pg, h, n_kv_heads, page_size, off, d_k, d)] =
                        orc_e4m3_code(load_elem(k_new, new_dtype, src) / (double)k_scale[h]);
                }
                for (int d = 0; d < d_v; ++d) {
                    size_t src = (((size_t)b * Q + i) * n_kv_heads + h) * d_v + d;
                    v_cache[gqa_index(pg, h, n_kv_heads, page_size, off, d_v, d)] =
                        orc_e4m3_code(load_elem(v_new, new_dtype, src) / (double)v_scale[h]);
                }
            }
        }
    }
    return ORC_OK;
}

/*
 * A tree of Q nodes per request in topological order: parent[0] = -1 and
 * 0 <= parent[i] < i for i >= 1.  Returns 1 if every request's tree is
 * well formed.
 */
int orc_tree_valid(int B, int Q, const int* parent) {
    for (int b = 0; b < B; ++b) {
        if (Q > 0 && parent[(size_t)b * Q] != -1) return 0;
        for (int i = 1; i < Q; ++i) {
            int p = parent[(size_t)b * Q + i];
            if (p < 0 || p >= i) return 0;
        }
    }
    return 1;
}

/*
 * Verify attention for the K+1 queries of each request, over a cache that
 * already holds the appended positions.  Query i of request b and head h
 * attends to keys 0 .. L_b+i (a causal mask over the K+1 new positions,
 * [TRT-MTP] "支持 MTP 的注意力機制"; the set of keys each draft sees follows
 * the table in [CSDN-MTP] step 2, with the query's own key included):
 *     s_p = scale * <q, k_p>,   o = sum_p softmax(s)_p * v_p
 * ([CSDN-MTP] step 2, Attention(Q_i) = Softmax(Q_i K^T / sqrt(d_k)) V).
 * GQA: query head h reads kv head floor(h * Hkv / Hq).
 * MLA: one latent vector per position; k_p = latent[0:d_qk] and
 * v_p = latent[0:d_v].
 *
 * FP8 cache (kv_dtype ORC_E4M3, GQA): k_p = code_value * k_scale[kv head] and
 * v_p = code_value * v_scale[kv head], elementwise; q stays in `dtype`.
 *
 * Tree of drafts (tree_parent, [B][Q], optional): the Q new positions are the
 * nodes of a tree in topological order, node 0 the root (parent -1) and
 * parent[i] < i for the others.  Node i attends to the cached keys 0 .. L_b-1
 * and to the new keys L_b + a for a = i and every ancestor of i -- the tree
 * attention mask that replaces the causal one when the drafts form a tree
 * ([TRT-MTP] "工作展望", Fig. 9: tree instead of chain drafting).  A chain
 * (parent[i] = i - 1) is the causal case.  An ill-formed tree is an
 * argument error.
 *
 * sel: n_sel triples (b, i, h) to evaluate, or NULL for every (b, i, h) in
 * that order.  out: [n_sel][d_v] doubles.
 */
int orc_verify_attn_ex(int B, int Q, int Hq, int Hkv, int d_qk, int d_v, int mla,
                       int page_size, int max_pages, int num_pages, double scale, int dtype,
                       int kv_dtype, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int* page_table,
                       const int* seq_lens, int n_sel, const int* sel, double* out,
                       const int* tree_parent) {
    if (kv_dtype == ORC_E4M3 && (mla || !k_scale || !v_scale)) return ORC_EARG;
    if (tree_parent && !orc_tree_valid(B, Q, tree_parent)) return ORC_EARG;
    long total = sel ? n_sel : (long)B * Q * Hq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
    for (long s = 0; s < total; ++s) {
        int b, i, h;
        if (sel) {
            b = sel[3 * s];
            i = sel[3 * s + 1];
            h = sel[3 * s + 2];
        } else {
            b = (int)(s / ((long)Q * Hq));
            i = (int)((s / Hq) % Q);
            h = (int)(s % Hq);
        }
        double* o = out + (size_t)s * d_v;
        if (b < 0 || b >= B || i < 0 || i >= Q || h < 0 || h >= Hq) {
            bad |= 1;
            continue;
        }
        long n = (long)seq_lens[b] + i + 1;  /* keys 0 .. L_b + i */
        long Lb = seq_lens[b];
        /* vis[a]: new key L_b + a is visible (chain: every a <= i) */
        unsigned char* vis = (unsigned char*)malloc((size_t)Q);
        for (int a = 0; a < Q; ++a) vis[a] = tree_parent ? 0 : (a <= i);
        if (tree_parent)
            for (int a = i; a >= 0; a = tree_parent[(size_t)b * Q + a]) vis[a] = 1;
        int kvh = mla ? 0 : (int)((long)h * Hkv / Hq);
        double ks = kv_dtype == ORC_E4M3 ? (double)k_scale[kvh] : 1.0;
        double vs = kv_dtype == ORC_E4M3 ? (double)v_scale[kvh] : 1.0;
        double* sc = (double*)malloc(sizeof(double) * (size_t)n);
        size_t qoff = (((size_t)b * Q + i) * Hq + h) * d_qk;
        double m = -INFINITY;
        for (long p = 0; p < n; ++p) {
            if (p >= Lb && !vis[p - Lb]) {
                sc[p] = -INFINITY;
                continue;
            }
            long pg = phys_page(page_table, max_pages, num_pages, b, p, page_size);
            if (pg < 0) {
                bad |= 2;
                sc[p] = -INFINITY;
                continue;
            }
            long off = p % page_size;
            double acc = 0.0;
            for (int d = 0; d < d_qk; ++d) {
                size_t ki = mla ? ((size_t)pg * page_size + off) * d_qk + d
                                : gqa_index(pg, kvh, Hkv, page_size, off, d_qk, d);
                acc += load_elem(q, dtype, qoff + d) * (load_elem(k_cache, kv_dtype, ki) * ks);
            }
            sc[p] = scale * acc;
            if (sc[p] > m) m = sc[p];
        }
        double denom = 0.0;
        for (long p = 0; p < n; ++p) {
            sc[p] = exp(sc[p] - m);
            denom += sc[p];
        }
        for (int d = 0; d < d_v; ++d) o[d] = 0.0;
        for (long p = 0; p < n; ++p) {
            if (p >= Lb && !vis[p - Lb]) continue;
            long pg = phys_page(page_table, max_pages, num_pages, b, p, page_size);
            if (pg < 0) continue;
            long off = p % page_size;
            for (int d = 0; d < d_v; ++d) {
                size_t vi = mla ? ((size_t)pg * page_size + off) * d_qk + d
                                : gqa_index(pg, kvh, Hkv, page_size, off, d_v, d);
                o[d] += sc[p] * (load_elem(mla ? k_cache : v_cache, kv_dtype, vi) * vs);
            }
        }
        for (int d = 0; d < d_v; ++d) o[d] /= denom;
        free(sc);
        free(vis);
    }
    return bad ? ORC_EPAGE : ORC_OK;
}

int orc_verify_attn(int B, int Q, int Hq, int Hkv, int d_qk, int d_v, int mla,
                    int page_size, int max_pages, int num_pages, double scale, int dtype,
                    const void* q, const void* k_cache, const void* v_cache,
                    const int* page_table, const int* seq_lens, int n_sel, const int* sel,
                    double* out) {
    return orc_verify_attn_ex(B, Q, Hq, Hkv, d_qk, d_v, mla, page_size, max_pages, num_pages,
                              scale, dtype, dtype, q, k_cache, v_cache, NULL, NULL, page_table,
                              seq_lens, n_sel, sel, out, NULL);
}

/*
 * LM head: logits[m][v] = sum_k H[m][k] * W[v][k], the output layer that maps
 * each position's hidden vector to vocabulary scores, all positions in one
 * product ([CSDN-MTP] step 4, Logits_i = H_i x W_o; W is stored one vocab row
 * per token, [V][hidden]).  Exact up to fp64 rounding of a sequential sum.
 * rows: n_rows row indices of H to evaluate (NULL: all M rows in order).
 * out: [n_rows][V] doubles.
 */
int orc_lm_head(int M, int hidden, int V, int dtype, const void* H, const void* W,
                int n_rows, const int* rows, double* out) {
    long nr = rows ? n_rows : M;
    long total = nr * (long)V;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < total; ++t) {
        long r = t / V;
        long v = t % V;
        long m = rows ? rows[r] : r;
        double acc = 0.0;
        for (int k = 0; k < hidden; ++k)
            acc += load_elem(H, dtype, (size_t)m * hidden + k) *
                   load_elem(W, dtype, (size_t)v * hidden + k);
        out[t] = acc;
    }
    (void)M;
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Acceptance.
 * ---------------------------------------------------------------------- */

/* Target token of a logits row under greedy decoding: the argmax, smallest
 * id among equal maxima.  Also returns the gap to the runner-up value (a
 * diagnostic: how close the decision was). */
static int row_argmax(const void* row, int dtype, int V, double* margin) {
    int best = 0;
    double bv = load_elem(row, dtype, 0);
    double second = -INFINITY;
    for (int v = 1; v < V; ++v) {
        double x = load_elem(row, dtype, v);
        if (x > bv) {
            second = bv;
            bv = x;
            best = v;
        } else if (x > second) {
            second = x;
        }
    }
    if (margin) *margin = bv - second;
    return best;
}

/* Greedy target token of each of n rows (smallest id among equal maxima,
 * [SD-PRACTICE] s4.4 argmax rule) and its margin over the runner-up. */
int orc_argmax_rows(int n, int V, int dtype, const void* logits, int* out, double* margin) {
    size_t es = elem_size(dtype);
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n; ++r)
        out[r] = row_argmax((const char*)logits + (size_t)r * V * es, dtype, V,
                            margin ? margin + r : NULL);
    return ORC_OK;
}

/* A row the acceptance rule can use: no NaN or +inf, not all -inf. */
static int row_valid(const void* row, int dtype, int V) {
    int finite = 0;
    for (int v = 0; v < V; ++v) {
        double x = load_elem(row, dtype, v);
        if (isnan(x) || x == INFINITY) return 0;
        if (x > -INFINITY) finite = 1;
    }
    return finite;
}

typedef struct {
    const void* row;
    int dtype;
} sort_ctx_t;
static sort_ctx_t g_sort_ctx; /* qsort has no context argument; guarded by
                                 the caller running single-threaded. */

static int cmp_desc(const void* a, const void* b) {
    int ia = *(const int*)a, ib = *(const int*)b;
    double xa = load_elem(g_sort_ctx.row, g_sort_ctx.dtype, ia);
    double xb = load_elem(g_sort_ctx.row, g_sort_ctx.dtype, ib);
    if (xa > xb) return -1;
    if (xa < xb) return 1;
    return (ia > ib) - (ia < ib);
}

/*
 * Target distribution of one row at temperature T > 0, with top-p:
 *   e_v = exp((l_v - max l) / T);
 *   top_p < 1: order tokens by (logit desc, id asc), take the shortest prefix
 *     whose mass sum(e)/Z reaches top_p, and keep every token whose logit is
 *     >= the last kept logit (ties are kept together);
 *   p_t(v) = keep(v) e_v / sum_{kept} e.
 * Writes p[V].  topp_gap: distance of top_p from the nearest achievable
 * prefix-mass boundary around the chosen threshold (diagnostic).
 */
static void row_target_probs(const void* row, int dtype, int V, double T, double top_p,
                             double* p, double* topp_gap) {
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double x = load_elem(row, dtype, v);
        if (x > m) m = x;
    }
    double Z = 0.0;
    for (int v = 0; v < V; ++v) {
        p[v] = exp((load_elem(row, dtype, v) - m) / T);
        Z += p[v];
    }
    double lambda = -INFINITY;
    if (topp_gap) *topp_gap = INFINITY;
    if (top_p < 1.0) {
        int* idx = (int*)malloc(sizeof(int) * (size_t)V);
        for (int v = 0; v < V; ++v) idx[v] = v;
        g_sort_ctx.row = row;
        g_sort_ctx.dtype = dtype;
        qsort(idx, (size_t)V, sizeof(int), cmp_desc);
        double cum = 0.0;
        int last = V - 1;
        for (int k = 0; k < V; ++k) {
            cum += p[idx[k]];
            if (cum >= top_p * Z) {
                last = k;
                break;
            }
        }
        lambda = load_elem(row, dtype, idx[last]);
        if (topp_gap) {
            /* Mass of the kept set, and mass strictly above its lowest level. */
            double above = 0.0, kept = 0.0;
            for (int v = 0; v < V; ++v) {
                double x = load_elem(row, dtype, v);
                if (x > lambda) above += p[v];
                if (x >= lambda) kept += p[v];
            }
            double g1 = fabs(kept / Z - top_p), g2 = fabs(above / Z - top_p);
            *topp_gap = g1 < g2 ? g1 : g2;
        }
        free(idx);
    }
    double Zk = 0.0;
    for (int v = 0; v < V; ++v) {
        if (load_elem(row, dtype, v) < lambda) p[v] = 0.0;
        Zk += p[v];
    }
    for (int v = 0; v < V; ++v) p[v] /= Zk;
}

/*
 * Inverse-CDF draw from weights r[0..V-1] (unnormalised, >= 0) with uniform
 * u: the smallest v whose running sum exceeds u * S, S = sum r, scanning in
 * token-id order.  If rounding leaves no such v, the largest v with r_v > 0.
 * edge: distance of u*S from the nearer edge of the chosen bucket, over S.
 */
static int inverse_cdf(const double* r, int V, double u, double* edge) {
    double S = 0.0;
    for (int v = 0; v < V; ++v) S += r[v];
    double target = u * S;
    double cum = 0.0;
    for (int v = 0; v < V; ++v) {
        double prev = cum;
        cum += r[v];
        if (cum > target) {
            if (edge) {
                double a = target - prev, b = cum - target;
                *edge = (a < b ? a : b) / S;
            }
            return v;
        }
    }
    if (edge) *edge = 0.0;
    for (int v = V - 1; v >= 0; --v)
        if (r[v] > 0) return v;
    return V - 1;
}

/*
 * Verify-and-accept for a batch of requests ([VLLM-MTP] s3 stage 3 and 4):
 *
 * Greedy (temperature 0; [SD-PRACTICE] s4.4): t_i = argmax of row i; draft n
 * is accepted while d_n == t_{n-1}; the first mismatch stops the chain and
 * all later drafts are discarded; the emitted tokens are the accepted drafts
 * followed by t_j ([TRT-MTP] Fig. 1: input G + drafts ABCDE, targets agree
 * on ABC, so A, B, C and the target's H are emitted).
 *
 * Stochastic (temperature > 0; [SD-PRACTICE] s2.3, s4.4; [VLLM-MTP] s3):
 * draft n is accepted iff u_accept[b][n-1] < min(1, p_t(d_n) / p_d(d_n)),
 * both distributions taken at row n-1; at the first rejection the chain
 * stops and the replacement token is drawn from norm(max(0, p_t - p_d)) of
 * row n-1 with u_sample[b][n-1]; if every draft is accepted the bonus token
 * is drawn from p_t of row K with u_sample[b][K] (1 .. K+1 tokens per
 * step, [VLLM-MTP] s3 stage 4).  A negative draft id ends the chain early
 * and the final token is drawn from p_t of that row.
 *
 * Invalid requests (temperature < 0 or NaN, top_p <= 0 or NaN when sampling,
 * sampling with K > 0 but no draft distribution, a draft id >= V, a row with NaN/+inf or no finite entry) emit nothing:
 * num_accepted = next_token = -1 and all out_tokens -1.
 *
 * Outputs: num_accepted[B] = j_b; out_tokens[B][K+1] (first j_b+1 valid,
 * rest -1); next_token[B] = the final token; out_offsets[B+1] exclusive
 * scan of emitted counts; packed[B*(K+1)] the emitted tokens back to back,
 * then -1.  diag[B][4] (optional): smallest top-2 logit margin over the
 * rows a greedy decision used; smallest |u - min(1, ratio)| over the
 * stochastic decisions taken; edge distance of the final draw; smallest
 * top-p boundary gap over the rows used.  Returns the count of invalid
 * requests.
 */
/*
 * Relaxed acceptance of one draft ([TRT-MTP] "寬松接受", Fig. 6): take the
 * top-N tokens of the row's logits (order: logit descending, id ascending),
 * compute the token probabilities with a softmax of the logits, drop every
 * candidate whose probability is below (top-1 probability - delta), and
 * accept the draft if it is one of the remaining candidates.  margin: the
 * draft's |p_d - (p_top1 - delta)| when it is among the top N (else
 * +inf).  Probabilities in fp64.
 */
int orc_accept_ex(int B, int K, int V, int logits_dtype, const void* logits,
                  const int* drafts, const float* temperature, const float* top_p,
                  const float* draft_probs, const float* u_accept, const float* u_sample,
                  const int* relaxed_topk, const float* relaxed_delta, int* num_accepted,
                  int* out_tokens, int* next_token, int* out_offsets, int* packed,
                  double* diag, const int* tree_parent, int* accepted_nodes);

static int relaxed_accepts(const void* row, int dtype, int V, int N, double delta, int d,
                           double* margin) {
    int* idx = (int*)malloc(sizeof(int) * (size_t)V);
    for (int v = 0; v < V; ++v) idx[v] = v;
    g_sort_ctx.row = row;
    g_sort_ctx.dtype = dtype;
    qsort(idx, (size_t)V, sizeof(int), cmp_desc);
    const int n_top = N < V ? N : V;
    double m = load_elem(row, dtype, idx[0]);
    double Z = 0.0;
    for (int v = 0; v < V; ++v) Z += exp(load_elem(row, dtype, v) - m);
    const double p_top1 = 1.0 / Z; /* exp(m - m) / Z */
    int hit = 0;
    *margin = INFINITY;
    for (int k = 0; k < n_top; ++k) {
        if (idx[k] != d) continue;
        const double p_d = exp(load_elem(row, dtype, d) - m) / Z;
        *margin = fabs(p_d - (p_top1 - delta));
        hit = !(p_d < p_top1 - delta);
    }
    free(idx);
    return hit;
}

int orc_accept(int B, int K, int V, int logits_dtype, const void* logits,
               const int* drafts, const float* temperature, const float* top_p,
               const float* draft_probs, const float* u_accept, const float* u_sample,
               int* num_accepted, int* out_tokens, int* next_token, int* out_offsets,
               int* packed, double* diag) {
    return orc_accept_ex(B, K, V, logits_dtype, logits, drafts, temperature, top_p, draft_probs,
                         u_accept, u_sample, NULL, NULL, num_accepted, out_tokens, next_token,
                         out_offsets, packed, diag, NULL, NULL);
}

/*
 * As orc_accept, plus relaxed acceptance for greedy requests:
 * relaxed_topk[b] > 0 (with relaxed_delta[b], finite and >= 0) replaces the
 * top-1 match of draft n by relaxed_accepts over row n-1 (the final token is
 * still the argmax of row j); 0 keeps the strict rule; sampled requests
 * ignore it.  A negative top-N, or a bad delta for a relaxed greedy request,
 * makes the request invalid.  Either array may be NULL (strict).  For
 * relaxed requests diag[1] holds the smallest margin of relaxed_accepts.
 *
 * Tree of drafts (tree_parent [B][K+1], optional; node 0 is the root, node
 * n >= 1 carries draft n, parent[n] < n): node n is accepted when its parent
 * is accepted (the root always is) and its draft equals the argmax of its
 * parent's row; the accepted nodes form a subtree holding the root, and the
 * verification keeps the longest accepted root-to-node path: the deepest
 * accepted node, the smallest node index among equally deep ones.  The
 * final token is the argmax of that node's row and the accepted drafts are
 * those along its path ([TRT-MTP] "工作展望", Fig. 9: a tree offers several
 * candidate continuations and the longest verified one is kept; a chain is
 * the case parent[n] = n - 1).  A negative draft id marks an unused node.
 * A malformed tree, a sampled request or a relaxed request with a tree is
 * invalid.  accepted_nodes [B][K+1] (optional, also without a tree) receives
 * the node path: 0, the accepted nodes, then -1.
 */
int orc_accept_ex(int B, int K, int V, int logits_dtype, const void* logits,
                  const int* drafts, const float* temperature, const float* top_p,
                  const float* draft_probs, const float* u_accept, const float* u_sample,
                  const int* relaxed_topk, const float* relaxed_delta, int* num_accepted,
                  int* out_tokens, int* next_token, int* out_offsets, int* packed,
                  double* diag, const int* tree_parent, int* accepted_nodes) {
    const int Q = K + 1;
    size_t es = elem_size(logits_dtype);
    int n_invalid = 0;
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    for (int b = 0; b < B; ++b) {
        const char* base = (const char*)logits + (size_t)b * Q * V * es;
        double T = temperature[b];
        double tp = top_p[b];
        double dg[4] = {INFINITY, INFINITY, INFINITY, INFINITY};
        int ok = !(isnan(T) || T < 0);
        if (ok && T > 0 && (isnan(tp) || tp <= 0)) ok = 0;
        const int rN = relaxed_topk ? relaxed_topk[b] : 0;
        const double rdelta = (relaxed_topk && relaxed_delta) ? relaxed_delta[b] : 0.0;
        if (rN < 0) ok = 0;
        if (ok && T == 0 && rN > 0 && (!relaxed_delta || !isfinite(rdelta) || rdelta < 0)) ok = 0;
        if (ok && T > 0 && K > 0 && !draft_probs) ok = 0;
        if (ok && tree_parent) {
            const int* par = tree_parent + (size_t)b * Q;
            if (!orc_tree_valid(1, Q, par) || T != 0.0 || rN > 0) ok = 0;
        }
        for (int n = 0; ok && n < K; ++n)
            if (drafts[(size_t)b * K + n] >= V) ok = 0;
        for (int i = 0; ok && i < Q; ++i)
            if (!row_valid(base + (size_t)i * V * es, logits_dtype, V)) ok = 0;
        for (int i = 0; i < Q; ++i) out_tokens[(size_t)b * Q + i] = -1;
        int* path = accepted_nodes ? accepted_nodes + (size_t)b * Q : NULL;
        if (path)
            for (int i = 0; i < Q; ++i) path[i] = i == 0 ? 0 : -1;
        if (!ok) {
            if (path) path[0] = -1;
            num_accepted[b] = -1;
            next_token[b] = -1;
            ++n_invalid;
            if (diag) memcpy(diag + 4 * (size_t)b, dg, sizeof dg);
            continue;
        }
        int j = 0, f = -1;
        if (tree_parent) {
            /* Every node's acceptance, in topological order (parents first),
             * then the deepest accepted node (smallest index on ties). */
            const int* par = tree_parent + (size_t)b * Q;
            int* acc = (int*)malloc(sizeof(int) * (size_t)Q);
            int* depth = (int*)malloc(sizeof(int) * (size_t)Q);
            int* amax = (int*)malloc(sizeof(int) * (size_t)Q);
            double mg;
            acc[0] = 1;
            depth[0] = 0;
            amax[0] = row_argmax(base, logits_dtype, V, &mg);
            dg[0] = mg;
            int best = 0;
            for (int n = 1; n < Q; ++n) {
                const int p = par[n], d = drafts[(size_t)b * K + n - 1];
                depth[n] = depth[p] + 1;
                acc[n] = acc[p] && d >= 0 && d == amax[p];
                amax[n] = -1;
                if (!acc[n]) continue;
                amax[n] = row_argmax(base + (size_t)n * V * es, logits_dtype, V, &mg);
                if (mg < dg[0]) dg[0] = mg;
                if (depth[n] > depth[best]) best = n;
            }
            j = depth[best];
            for (int c = best; c != 0; c = par[c]) {
                if (path) path[depth[c]] = c;
                out_tokens[(size_t)b * Q + depth[c] - 1] = drafts[(size_t)b * K + c - 1];
            }
            f = amax[best];
            free(acc);
            free(depth);
            free(amax);
        } else if (T == 0.0 && rN > 0) {
            /* Relaxed: draft n is accepted while it is a surviving top-N
             * candidate of row n-1; the final token is the argmax of row j. */
            while (j < K) {
                int d = drafts[(size_t)b * K + j];
                if (d < 0) break;
                double mr;
                int hit = relaxed_accepts(base + (size_t)j * V * es, logits_dtype, V, rN, rdelta,
                                          d, &mr);
                if (mr < dg[1]) dg[1] = mr;
                if (!hit) break;
                ++j;
            }
            double mg;
            f = row_argmax(base + (size_t)j * V * es, logits_dtype, V, &mg);
            dg[0] = mg;
        } else if (T == 0.0) {
            double mg;
            int t = row_argmax(base, logits_dtype, V, &mg);
            dg[0] = mg;
            while (j < K) {
                int d = drafts[(size_t)b * K + j];
                if (d < 0 || d != t) break;
                ++j;
                t = row_argmax(base + (size_t)j * V * es, logits_dtype, V, &mg);
                if (mg < dg[0]) dg[0] = mg;
            }
            f = t;
        } else {
            j = K;
            for (int n = 1; n <= K; ++n) {
                const void* row = base + (size_t)(n - 1) * V * es;
                double gap;
                row_target_probs(row, logits_dtype, V, T, tp, pt, &gap);
                if (gap < dg[3]) dg[3] = gap;
                int d = drafts[(size_t)b * K + n - 1];
                double u_s = u_sample[(size_t)b * Q + n - 1];
                if (d < 0) {
                    j = n - 1;
                    f = inverse_cdf(pt, V, u_s, &dg[2]);
                    break;
                }
                const float* pd = draft_probs + ((size_t)b * K + n - 1) * V;
                double a = pt[d], qd = pd[d];
                double ratio = qd > 0 ? a / qd : (a > 0 ? INFINITY : 0.0);
                double acc_p = ratio < 1.0 ? ratio : 1.0;
                double u = u_accept[(size_t)b * Q + n - 1];
                if (fabs(u - acc_p) < dg[1]) dg[1] = fabs(u - acc_p);
                if (u < acc_p) continue;
                j = n - 1;
                double S = 0.0;
                for (int v = 0; v < V; ++v) {
                    double x = pt[v] - (double)pd[v];
                    r[v] = x > 0 ? x : 0.0;
                    S += r[v];
                }
                f = inverse_cdf(S > 0 ? r : pt, V, u_s, &dg[2]);
                break;
            }
            if (f < 0) {
                double gap;
                row_target_probs(base + (size_t)K * V * es, logits_dtype, V, T, tp, pt, &gap);
                if (gap < dg[3]) dg[3] = gap;
                f = inverse_cdf(pt, V, u_sample[(size_t)b * Q + K], &dg[2]);
            }
        }
        num_accepted[b] = j;
        next_token[b] = f;
        if (!tree_parent) {
            for (int n = 0; n < j; ++n) out_tokens[(size_t)b * Q + n] = drafts[(size_t)b * K + n];
            if (path)
                for (int n = 1; n <= j; ++n) path[n] = n;
        }
        out_tokens[(size_t)b * Q + j] = f;
        if (diag) memcpy(diag + 4 * (size_t)b, dg, sizeof dg);
    }
    free(pt);
    free(r);
    out_offsets[0] = 0;
    for (int b = 0; b < B; ++b)
        out_offsets[b + 1] = out_offsets[b] + (num_accepted[b] >= 0 ? num_accepted[b] + 1 : 0);
    for (size_t k = 0; k < (size_t)B * Q; ++k) packed[k] = -1;
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < out_offsets[b + 1] - out_offsets[b]; ++k)
            packed[out_offsets[b] + k] = out_tokens[(size_t)b * Q + k];
    return n_invalid;
}

/*
 * KV rollback ([TRT-MTP] "MTP Vanilla"/"MTP Eagle": the keys/values of
 * discarded drafts are cleared from the cache; "基本實現方式": this is done
 * after the engine forward; [CSDN-MTP] rollback keeps the verified prefix
 * and recomputes nothing).  After the step, request b keeps its old L_b
 * positions plus the root and the j_b accepted drafts:
 *     new_len = L_b + j_b + 1;
 * positions new_len .. L_b+K are rejected.  An invalid j_b (< 0 or > K)
 * keeps nothing of the step: new_len = L_b and L_b .. L_b+K are rejected.
 * Outputs, compacted in (request, position) order:
 *   rb_slots: physical slot page*page_size + offset of each rejected
 *             position, rb_offsets[B+1] its per-request offsets;
 *   freed:    the physical page of every logical page the step wrote to that
 *             now holds no kept position (logical page >= ceil(new_len /
 *             page_size)), freed_offsets[B+1].
 * seq_lens is updated in place.  If poison is set, the rejected slots of the
 * caches (every kv head; the latent row for MLA) are zeroed.
 * Tree of drafts: accepted_nodes [B][K+1] (optional) is the accepted node
 * path of each request (0, the j_b accepted nodes in increasing order, then
 * -1).  Node a was appended at slot L_b + a, so the kept positions are not
 * contiguous; the cache rows of slot L_b + path[t] are copied to slot
 * L_b + t for t = 1 .. j_b, in increasing t (a destination is never a later
 * source, since path[t] >= t), before any poisoning.  A path that does not
 * start at 0, is not increasing or leaves 0 .. K counts as an invalid j_b.
 * Returns the count of invalid j_b.
 */
int orc_kv_rollback(int B, int K, int page_size, int max_pages, const int* page_table,
                    const int* num_accepted, int* seq_lens, int* rb_slots, int* rb_offsets,
                    int* freed, int* freed_offsets, int poison, int n_kv_heads, int d_k,
                    int d_v, int mla, int dtype, void* k_cache, void* v_cache,
                    const int* accepted_nodes) {
    int n_bad = 0;
    size_t es = elem_size(dtype);
    rb_offsets[0] = 0;
    freed_offsets[0] = 0;
    for (int b = 0; b < B; ++b) {
        long L = seq_lens[b];
        int j = num_accepted[b];
        long new_len;
        const int* path = accepted_nodes ? accepted_nodes + (size_t)b * (K + 1) : NULL;
        int path_ok = 1;
        if (path && j >= 0 && j <= K) {
            if (path[0] != 0) path_ok = 0;
            for (int t = 1; t <= j && path_ok; ++t)
                if (path[t] <= path[t - 1] || path[t] > K) path_ok = 0;
        }
        if (j < 0 || j > K || !path_ok) {
            ++n_bad;
            new_len = L;
        } else {
            new_len = L + j + 1;
        }
        if (path && new_len > L && (k_cache || v_cache)) {
            for (int t = 1; t <= j; ++t) {
                if (path[t] == t) continue;
                long ps = L + path[t], pd = L + t;
                long gs = page_table[(size_t)b * max_pages + ps / page_size];
                long gd = page_table[(size_t)b * max_pages + pd / page_size];
                long os = ps % page_size, od = pd % page_size;
                if (mla) {
                    memmove((char*)k_cache + ((size_t)gd * page_size + od) * d_k * es,
                            (char*)k_cache + ((size_t)gs * page_size + os) * d_k * es,
                            (size_t)d_k * es);
                    continue;
                }
                for (int h = 0; h < n_kv_heads; ++h) {
                    memmove((char*)k_cache + gqa_index(gd, h, n_kv_heads, page_size, od, d_k, 0) * es,
                            (char*)k_cache + gqa_index(gs, h, n_kv_heads, page_size, os, d_k, 0) * es,
                            (size_t)d_k * es);
                    memmove((char*)v_cache + gqa_index(gd, h, n_kv_heads, page_size, od, d_v, 0) * es,
                            (char*)v_cache + gqa_index(gs, h, n_kv_heads, page_size, os, d_v, 0) * es,
                            (size_t)d_v * es);
                }
            }
        }
        int ns = 0;
        for (long p = new_len; p <= L + K; ++p) {
            long pg = page_table[(size_t)b * max_pages + p / page_size];
            long off = p % page_size;
            rb_slots[rb_offsets[b] + ns] = (int)(pg * page_size + off);
            ++ns;
            if (poison) {
                if (mla) {
                    memset((char*)k_cache + ((size_t)pg * page_size + off) * d_k * es, 0,
                           (size_t)d_k * es);
                } else {
                    for (int h = 0; h < n_kv_heads; ++h) {
                        memset((char*)k_cache +
                                   gqa_index(pg, h, n_kv_heads, page_size, off, d_k, 0) * es,
                               0, (size_t)d_k * es);
                        memset((char*)v_cache +
                                   gqa_index(pg, h, n_kv_heads, page_size, off, d_v, 0) * es,
                               0, (size_t)d_v * es);
                    }
                }
            }
        }
        rb_offsets[b + 1] = rb_offsets[b] + ns;
        long first_free = (new_len + page_size - 1) / page_size;
        long first_touched = L / page_size, last_touched = (L + K) / page_size;
        int nf = 0;
        for (long lp = first_touched; lp <= last_touched; ++lp) {
            if (lp < first_free) continue;
            freed[freed_offsets[b] + nf] = page_table[(size_t)b * max_pages + lp];
            ++nf;
        }
        freed_offsets[b + 1] = freed_offsets[b] + nf;
        seq_lens[b] = (int)new_len;
    }
    return n_bad;
}
