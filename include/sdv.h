/*
 * sdv.h -- C ABI of the MI355X (gfx950) speculative-decoding verify step.
 *
 * One verify step of a draft chain runs four calls on one HIP stream:
 *   sd_verify_attn   append the K+1 new keys/values, causal attention of the
 *                    root token plus K drafts over the paged KV cache
 *   sd_lm_head       project every position's hidden vector to vocab logits
 *   sd_accept        greedy longest-prefix match or rejection sampling, with
 *                    the correction/bonus token and a packed token list
 *   sd_kv_rollback   drop the rejected positions from the cache bookkeeping
 *
 * Pages cited (titles and sections; the text is Chinese):
 *   [TRT-MTP]     TensorRT-LLM MTP implementation/optimisation article
 *                 (makelele.cn/d/6983435): "背景" Fig. 1, "MTP Vanilla",
 *                 "MTP Eagle", "基本實現方式" Fig. 4, "支持 MTP 的注意力機制".
 *   [SD-PRACTICE] "推测解码与MTP：大模型推理加速的核心技术与工程实践"
 *                 (mlqm.cn/news/1017475): s2.2, s2.3, s4.3, s4.4.
 *   [CSDN-MTP]    CSDN article on the two meanings of "MTP"
 *                 (gitcode.csdn.net/69b64a3354b52172bc617fab): "整体计算流程
 *                 （以 K=3 草稿 Token 为例）" steps 2, 4, 5, 6; "回滚机制".
 *   [VLLM-MTP]    "MPT (MTP, Multi-Token Prediction) 原理详解"
 *                 (mqxn.cn/news/75683): s3 stages 3-4, s4, s5.
 *
 * Conventions shared by every call
 *   - Pointers marked "device" are HIP device pointers; descriptors and size
 *     outputs are host memory.  The caller owns every buffer; the library
 *     allocates nothing and keeps no pointer after a call returns.
 *   - Every call but sd_get_device_error is asynchronous on `stream` (a
 *     hipStream_t; NULL = the default stream) and never synchronises the
 *     host.  Buffers must stay alive until the stream has passed the call.
 *   - Arrays are dense and row-major; element counts, not bytes, unless
 *     stated.  Tensor data pointers must be 16-byte aligned; workspaces
 *     256-byte aligned.
 *   - Status codes: arguments are checked on the host before anything is
 *     launched (SD_EINVAL, SD_EUNSUPPORTED, SD_EWORKSPACE); SD_EDEVICE
 *     reports a HIP launch error.  sd_last_error() returns this thread's
 *     text for the last non-OK status.  No exception crosses the ABI.
 *   - Faults only the device can see (a bad page-table entry, a sequence
 *     over capacity, an out-of-range draft id, non-finite logits, bad
 *     sampling parameters) are OR-ed as SD_DERR_* bits into the optional
 *     device int `dev_error` (clear it to 0 before the step) and make the
 *     offending request produce the documented "invalid" outputs; the
 *     kernels never read or write outside the buffers described here.
 *   - Calls hold no global mutable state and are re-entrant across streams
 *     when given distinct workspaces.
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SD_ABI_VERSION 5

/* status codes */
#define SD_OK 0
#define SD_EINVAL 1
#define SD_EUNSUPPORTED 2
#define SD_EWORKSPACE 3
#define SD_EDEVICE 4

/* element types */
#define SD_F32 0
#define SD_BF16 1
#define SD_E4M3 2   /* OCP 8-bit float E4M3, "fn" variant (KV caches only) */

/* KV cache formats (sd_attn_desc.kv_format) */
#define SD_KV_AS_DTYPE 0   /* k_cache / v_cache hold `dtype` elements */
#define SD_KV_E4M3 1       /* k_cache / v_cache hold SD_E4M3 codes, scaled per kv head */

/* attention layouts */
#define SD_ATTN_GQA 0
#define SD_ATTN_MLA 1

/* device error bits */
#define SD_DERR_PAGE 1          /* a page-table entry the step needs is out of range */
#define SD_DERR_CAPACITY 2      /* L_b < 0, L_b > max_seq_len, or L_b+K+1 > max_pages*page_size */
#define SD_DERR_TOKEN 4         /* a draft id >= vocab */
#define SD_DERR_NONFINITE 8     /* a logits row with NaN/+inf or no finite entry */
#define SD_DERR_PARAM 16        /* temperature < 0 or NaN; top_p <= 0 or NaN while sampling;
                                   sampling with K > 0 but no draft_probs */
#define SD_DERR_ACCEPT_COUNT 32 /* rollback given num_accepted > K */
#define SD_DERR_TREE 64         /* a malformed draft tree (parent[0] != -1 or parent[i]
                                   outside 0 .. i-1), a tree on a sampled or relaxed
                                   request, or a malformed accepted-node path */

/* Version of this header the library was built from (SD_ABI_VERSION). */
int sd_abi_version(void);

/* Text of this thread's last non-OK status ("" if none).  Valid until the
 * thread's next call into the library. */
const char* sd_last_error(void);

/* Device-side error report of a step ([VLLM-MTP] s3 stages 3-4: a verify
 * step ends with 1 .. D+1 tokens per request; a request the kernels had to
 * declare invalid ends with none, and this word says why).
 *   dev_error  device int32: the word passed as `dev_error` to the step's
 *              sd_verify_attn / sd_accept / sd_kv_rollback calls, into which
 *              they OR their SD_DERR_* bits (0 = no device-side fault)
 *   code       host int32, receives the word
 *   stream     the stream those calls were issued on (NULL = default)
 * Waits until `stream` has passed every call issued on it before this one,
 * then copies the word to *code.  It is the one call that synchronises the
 * host.  The word is not cleared: the caller zeroes it before the next
 * step.  Returns SD_EINVAL for a NULL pointer, SD_EDEVICE (code untouched)
 * if the copy or the wait fails. */
int sd_get_device_error(const int32_t* dev_error, int32_t* code, void* stream);

/* ------------------------------------------------------------------------
 * Verify attention.
 * [TRT-MTP] "支持 MTP 的注意力機制": in generation the chain gives K+1 input
 * tokens per request and a causal mask over them is all the attention needs.
 * [CSDN-MTP] step 2: the queries of the new tokens are batched into one
 * matrix against the cached keys, softmax(Q K^T / sqrt(d_k)) V, and each
 * new key/value is written into the cache as it is produced.
 *
 * For request b with cached length L_b = seq_lens[b]:
 *   1. k_new/v_new row i is written to position L_b+i (i = 0..K) of the
 *      paged cache (skipped when k_new is NULL: already appended);
 *   2. query i of head h attends to positions 0 .. L_b+i (its own key
 *      included):  out = softmax(scale * q k^T) v.
 * seq_lens is read only; sd_kv_rollback advances it.
 *
 * Layouts (device; dtype = SD_BF16 or SD_F32 for q, k_new, v_new, caches):
 *   q          [B][K+1][n_q_heads][d_qk]
 *   GQA: k_new [B][K+1][n_kv_heads][d_qk],  v_new [B][K+1][n_kv_heads][d_v]
 *        k_cache [num_pages][n_kv_heads][page_size][d_qk]
 *        v_cache [num_pages][n_kv_heads][page_size][d_v]
 *        query head h reads kv head h / (n_q_heads / n_kv_heads)
 *   MLA: one latent row per position shared by every head; k_new
 *        [B][K+1][d_qk], k_cache [num_pages][page_size][d_qk]; keys are the
 *        whole latent row, values its first d_v entries; v_new and v_cache
 *        must be NULL, n_kv_heads must be 1
 *   page_table int32 [B][max_pages]: logical page p/page_size of request b
 *        -> physical page; entries past the step's last position are unread
 *   seq_lens   int32 [B]
 *   out        float32 [B][K+1][n_q_heads][d_v]
 *   out_lowp   optional, out rounded to nearest-even in `dtype`, laid out
 *              [B*(K+1)][n_q_heads*d_v] (ready as LM-head input); may be NULL
 * A request with a capacity or page-table fault gets NaN outputs.
 *
 * Tree of drafts (tree_parent != NULL; [TRT-MTP] "工作展望", Fig. 9: tree
 * drafting instead of a chain).  The K+1 new positions of request b are the
 * nodes of a tree in topological order: node 0 is the root (parent -1),
 * every other node i has parent tree_parent[b][i] in 0 .. i-1.  Node i is
 * still appended at position L_b+i, and query i attends to positions
 * 0 .. L_b-1 and to L_b+a for a = i and every ancestor a of i (the causal
 * rule is the chain parent[i] = i-1).  A malformed tree makes the request
 * invalid (SD_DERR_TREE, NaN outputs).  Needs K+1 <= 64; GQA (either cache
 * format) and the float32 path only.
 *
 * FP8 KV cache (kv_format = SD_KV_E4M3; GQA with dtype SD_BF16 only).  The
 * pages name FP8 attention kernels as prior art for this step ([TRT-MTP]
 * "支持 MTP 的注意力機制"); the format here is OCP E4M3 ("fn": bias 7, no
 * infinities, 0x7F/0xFF NaN, largest finite 448), one byte per element in
 * the same [num_pages][n_kv_heads][page_size][d] layouts.  Element d of kv
 * head h stands for value(code) * k_scale[h] (keys) or value(code) *
 * v_scale[h] (values); k_scale, v_scale: device float32 [n_kv_heads],
 * positive and finite (other values are the caller's error: outputs are
 * then meaningless, but no access leaves the buffers).  The append stores
 * the code nearest to bf16_value / scale[h] (float32 division, correctly
 * rounded; ties to the even code; magnitudes above 448, infinities
 * included, saturate to 448; NaN -> 0x7F).  q, k_new, v_new, out_lowp stay
 * bf16.  The attention computes with the exact code values (every E4M3
 * value is a bf16 and an fp16 value) and applies the scales in float32; the
 * softmax weights meet the values rounded to fp16 (relative error at most
 * 2^-11 per weight), so an output element may differ from exact arithmetic
 * on the codes by up to 2^-11 of the weighted mean of |v| (measured: below
 * 6e-4 of the row's largest output; the bf16 cache path is exact to about
 * 1e-5).
 *
 * Supported: page_size 64; GQA bf16 (bf16 or E4M3 cache) with d_qk = d_v in
 * {64, 128} and (n_q_heads/n_kv_heads)*(K+1) <= 64; GQA f32 with d_qk = d_v
 * a divisor of 256 and a multiple of 4 (whole 16-byte rows); MLA bf16 with
 * d_qk = 576, d_v = 512 and n_q_heads a multiple of 32.  Others return
 * SD_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
typedef struct sd_attn_desc {
    int batch;
    int num_q;          /* K + 1 */
    int n_q_heads;
    int n_kv_heads;
    int d_qk;
    int d_v;
    int kind;           /* SD_ATTN_GQA or SD_ATTN_MLA */
    int dtype;          /* SD_F32 or SD_BF16 */
    int page_size;
    int max_pages;      /* row length of page_table */
    int num_pages;      /* pages in the physical pool */
    int max_seq_len;    /* host upper bound on every L_b (sizes the launch) */
    float softmax_scale;/* 0 selects 1/sqrt(d_qk) */
    const void* q;
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int32_t* page_table;
    const int32_t* seq_lens;
    float* out;
    void* out_lowp;
    int32_t* dev_error; /* optional */
    int kv_format;          /* SD_KV_AS_DTYPE (0) or SD_KV_E4M3 */
    const float* k_scale;   /* SD_KV_E4M3: device [n_kv_heads]; else unread */
    const float* v_scale;   /* SD_KV_E4M3: device [n_kv_heads]; else unread */
    const int32_t* tree_parent; /* optional device [B][K+1]; NULL = chain (ABI version 4) */
} sd_attn_desc;

/* Bytes of device workspace sd_verify_attn needs for this descriptor
 * (depends on shapes and max_seq_len only). */
int sd_verify_attn_workspace_size(const sd_attn_desc* d, size_t* bytes);

/* Runs the append and the attention.  workspace: device, >= the size above,
 * 256-byte aligned, contents need no initialisation. */
int sd_verify_attn(const sd_attn_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * LM head.  [CSDN-MTP] step 4: the hidden vectors of all verified positions
 * are stacked into one matrix and multiplied by the output-layer weights,
 * mapping hidden size to vocabulary size: logits = H x W_o.
 *   H      device [M][hidden]      (M = B*(K+1) rows)
 *   W      device [vocab][hidden]  (one row per token)
 *   logits device [M][vocab]; every element is sum_k H[m][k] W[v][k]
 *          accumulated in float32 and stored in `dtype` (bf16: round to
 *          nearest even).
 * dtype: SD_BF16 or SD_F32 for all three.  hidden must be a multiple of 8.
 * ---------------------------------------------------------------------- */
int sd_lm_head(int M, int hidden, int vocab, int dtype, const void* H, const void* W,
               void* logits, void* stream);

/* ------------------------------------------------------------------------
 * Acceptance.  [VLLM-MTP] s3 stages 3-4; [SD-PRACTICE] s2.3, s4.4;
 * [TRT-MTP] Fig. 1.  Logits row i of request b predicts position i+1; draft
 * n (1-based) is judged by row n-1.
 *
 * Greedy (temperature[b] == 0): t_i = argmax of row i, smallest id on ties;
 *   draft n is accepted while d_n == t_{n-1}; the first mismatch ends the
 *   chain; the final token is t_j.
 * Sampling (temperature[b] > 0): p_t of row i is softmax(l / T) restricted,
 *   when top_p[b] < 1, to the shortest prefix of tokens ordered by (logit
 *   desc, id asc) whose mass reaches top_p, extended to every token tied
 *   with the prefix's last logit, and renormalised.  Draft n is accepted
 *   iff u_accept[b][n-1] < min(1, p_t(d_n) / p_d(d_n)) (row n-1 of both;
 *   p_d = 0 counts as ratio +inf when p_t > 0, 0 when p_t = 0).  At the
 *   first rejection the final token is drawn from norm(max(0, p_t - p_d))
 *   of row n-1 (from p_t if that residual is all zero); if every draft is
 *   accepted it is drawn from p_t of row K.  Draws take the smallest v whose
 *   running sum over token ids exceeds u_sample[b][row] * (total); the
 *   statistics and sums are kept in float64.
 * Relaxed greedy verification ([TRT-MTP] "寬松接受", Fig. 6): with
 *   relaxed_topk[b] = N > 0 and temperature[b] == 0, draft n is accepted
 *   while it is one of the N largest logits of row n-1 (order: logit desc,
 *   id asc) and its softmax probability (T = 1, fp64) is not below the
 *   top-1 probability minus relaxed_delta[b]; the final token is still the
 *   argmax of row j.  N = 0 keeps the strict rule; sampled requests ignore
 *   N.  N < 0, or (for a relaxed greedy request) a delta that is NaN,
 *   infinite or negative, makes the request invalid (SD_DERR_PARAM).
 * A draft id < 0 ends the chain early (the final token is then drawn from,
 *   or is the argmax of, the row that draft would have been judged by).
 * Tree of drafts (tree_parent != NULL, the same array as sd_attn_desc's;
 *   [TRT-MTP] "工作展望", Fig. 9): node n >= 1 carries draft n and logits
 *   row n is the prediction after node n.  Node n is accepted when its
 *   parent is (the root always is) and its draft equals the argmax of the
 *   parent's row.  The kept path is the longest accepted root-to-node path:
 *   it ends at the deepest accepted node, the one with the smallest index
 *   among equally deep ones.  The final token is the argmax of that node's
 *   row; the emitted tokens are the drafts along the path, then the final
 *   token.  A negative draft id marks an unused node.  Trees apply to strict
 *   greedy requests only: a sampled or relaxed request with a tree, or a
 *   malformed tree, is invalid (SD_DERR_TREE).  Needs K+1 <= 64.
 * Each request emits j_b + 1 tokens: accepted drafts, then the final token.
 *
 * Layouts (device):
 *   logits       [B][K+1][vocab], logits_dtype SD_BF16 or SD_F32
 *   draft_tokens int32 [B][K]
 *   temperature  float32 [B]
 *   top_p        float32 [B], or NULL: no nucleus filtering for any request
 *   draft_probs  float32 [B][K][vocab] (row n-1 is the draft distribution
 *                draft n was drawn from), or NULL when every request is greedy
 *                or K == 0
 *   u_accept, u_sample  float32 [B][K+1], uniforms in [0, 1)
 *   relaxed_topk int32 [B], relaxed_delta float32 [B]: both NULL (strict
 *                for every request) or relaxed_topk set; relaxed_delta is
 *                read for greedy requests with relaxed_topk[b] > 0
 * Outputs (device):
 *   num_accepted int32 [B]         j_b, or -1 for an invalid request
 *   out_tokens   int32 [B][K+1]    j_b+1 emitted tokens, then -1
 *   next_token   int32 [B]         the final token (or -1)
 *   out_offsets  int32 [B+1]       exclusive scan of emitted counts
 *   packed_tokens int32 [B*(K+1)]  emitted tokens back to back, then -1
 *   accepted_nodes int32 [B][K+1]  optional: the accepted node path (0, the
 *                  accepted nodes, then -1; a chain gives 0 .. j_b; all -1
 *                  for an invalid request), the input sd_kv_rollback
 *                  gathers a tree's kept rows with
 * Invalid requests (see SD_DERR_TOKEN/NONFINITE/PARAM/TREE) emit nothing.
 * Returns SD_EINVAL for NULL required pointers, batch < 1, K < 0, vocab < 1
 * or an unknown logits dtype, and SD_EUNSUPPORTED for vocab > 262144 or a
 * tree with K+1 > 64.
 * ---------------------------------------------------------------------- */
typedef struct sd_accept_desc {
    int batch;
    int K;
    int vocab;
    int logits_dtype;
    const void* logits;
    const int32_t* draft_tokens;
    const float* temperature;
    const float* top_p;
    const float* draft_probs;
    const float* u_accept;
    const float* u_sample;
    int32_t* num_accepted;
    int32_t* out_tokens;
    int32_t* next_token;
    int32_t* out_offsets;
    int32_t* packed_tokens;
    int32_t* dev_error; /* optional */
    const int32_t* relaxed_topk;  /* optional (ABI version 2) */
    const float* relaxed_delta;   /* optional (ABI version 2) */
    const int32_t* tree_parent;   /* optional (ABI version 4) */
    int32_t* accepted_nodes;      /* optional output (ABI version 4) */
} sd_accept_desc;

int sd_accept_workspace_size(const sd_accept_desc* d, size_t* bytes);

/* workspace: device, >= sd_accept_workspace_size, 256-byte aligned. */
int sd_accept(const sd_accept_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* Allocation-free sd_accept, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same descriptor, outputs and semantics as sd_accept; the row
 * statistics and draw sums live in a fixed 4 MiB device array of the library
 * instead of a caller workspace (one copy per GPU, held until the process
 * ends).  That holds about 136 bytes per logits row (B*(K+1)) plus 32 bytes
 * per 512 vocabulary ids of each request: about 30000 rows for a small
 * vocabulary, 495 requests at K = 4 and V = 129280.  A batch beyond it gets
 * SD_EWORKSPACE before anything is launched.  Every call on one GPU
 * uses that GPU's one array, so calls that overlap on one GPU (on different
 * streams, or from host threads without an order between them) race: the
 * caller serialises them.  The first call on a device looks the array's
 * address up (hipGetSymbolAddress) with that device current; no call
 * allocates or frees memory. */
int sd_accept_noalloc(const sd_accept_desc* d, void* stream);

/* ------------------------------------------------------------------------
 * KV rollback.  [TRT-MTP] "MTP Vanilla"/"MTP Eagle": the keys/values of
 * discarded drafts are cleared so later steps stay correct; "基本實現方式"
 * Fig. 4: rollback is the one step run outside the engine forward.
 * [CSDN-MTP] "回滚机制": the verified prefix is kept and nothing is
 * recomputed.
 *
 * new_len = L_b + j_b + 1 (the root and the j_b accepted drafts stay).
 * Positions new_len .. L_b+K are rejected.  j_b < 0 (an invalid request)
 * keeps nothing of the step (new_len = L_b); j_b > K is treated the same
 * and sets SD_DERR_ACCEPT_COUNT.
 *
 *   page_table   int32 [B][max_pages]  (read)
 *   num_accepted int32 [B]             (read)
 *   seq_lens     int32 [B]             (read L_b, write new_len)
 *   rollback_slots   int32 [B*(K+1)]: physical slot page*page_size+offset
 *                    of every rejected position, in (request, position)
 *                    order; entries past the total are -1
 *   rollback_offsets int32 [B+1]
 *   freed_pages      int32 [B*(K/page_size+2)]: physical pages of the
 *                    logical pages the step wrote that hold no kept position
 *                    (logical page >= ceil(new_len/page_size)), in (request,
 *                    logical page) order; entries past the total are -1
 *   freed_offsets    int32 [B+1]
 *   poison_rejected: when non-zero, the rejected slots of k_cache/v_cache
 *                    (every kv head; the latent row for MLA) are zeroed;
 *                    kind, dtype, n_kv_heads, d_k, d_v describe the caches
 *                    as in sd_attn_desc (dtype = the cache element type:
 *                    SD_F32, SD_BF16, or SD_E4M3 for an FP8 cache, whose
 *                    zero code is +0) and are read only then (and for a
 *                    tree gather).
 *   accepted_nodes:  optional int32 [B][K+1], the path sd_accept returned for
 *                    a tree of drafts.  Node a was appended at L_b + a, so the
 *                    kept drafts are not contiguous: before anything else the
 *                    cache rows of position L_b + path[t] are copied to
 *                    L_b + t for t = 1 .. j_b (every kv head; the latent row
 *                    for MLA), in increasing t.  A path that does not start
 *                    at 0, does not increase or leaves 0 .. K keeps nothing
 *                    (new_len = L_b) and sets SD_DERR_TREE.  Needs the cache
 *                    description.
 * The page table itself is left unchanged: the caller returns freed pages
 * to its pool.
 * ---------------------------------------------------------------------- */
typedef struct sd_rollback_desc {
    int batch;
    int K;
    int page_size;
    int max_pages;
    const int32_t* page_table;
    const int32_t* num_accepted;
    int32_t* seq_lens;
    int32_t* rollback_slots;
    int32_t* rollback_offsets;
    int32_t* freed_pages;
    int32_t* freed_offsets;
    int poison_rejected;
    int kind;
    int dtype;
    int n_kv_heads;
    int d_k;
    int d_v;
    int num_pages;
    void* k_cache;
    void* v_cache;
    int32_t* dev_error; /* optional */
    const int32_t* accepted_nodes; /* optional (ABI version 4) */
} sd_rollback_desc;

int sd_kv_rollback(const sd_rollback_desc* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDV_H */
