/*
 * mla_decode.h - C ABI of a gfx950 (MI355X) library for weight-absorbed
 * Multi-head Latent Attention (MLA) decode over a paged latent KV cache.
 *
 * What is computed (each entry point below cites the passage it implements):
 *
 *   For query row n of request b and head h, with cache rows c_t of the
 *   request's tokens t < L_b (each row: 512 latent values, then 64 rope values):
 *     s_t   = sm_scale * (q_nope[n,h,:] . c_t[0:512] + q_rope[n,h,:] . c_t[512:576])
 *     out   = sum_t softmax(s)_t * c_t[0:512]        (the latent is also the value)
 *     lse   = ln sum_t exp(s_t)                      (natural log)
 *   q_nope is the absorbed query: the per-head no-rope query already multiplied
 *   by W_UK, as in section 2.1 of the sglang-jax MLA gap page and the forward
 *   path of the SGLang v0.3 MLA page. The two-path score, the online softmax
 *   and the latent-as-value product are the core loop of the MLA kernel in
 *   section 2.4 of the gap page.
 *
 * Conventions shared by every entry point:
 *   - Every pointer named *_d is device memory; *_h is host memory. The caller
 *     owns all memory. The library allocates nothing and never synchronises
 *     the device; all device work is enqueued on the caller's stream, passed as
 *     a hipStream_t cast to void* (NULL = the null stream).
 *   - Arguments are validated on the host before anything is enqueued. A
 *     non-zero return means nothing was enqueued (MLA_ERR_HIP aside: a launch
 *     the runtime rejected).
 *   - The library holds no state besides a cached device-property query.
 *   - Calls that share a workspace and overlap on different streams race.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,         /* NULL pointer, bad size, malformed CSR arrays */
    MLA_ERR_UNSUPPORTED = 2,         /* a shape or dtype the library does not implement */
    MLA_ERR_WORKSPACE_TOO_SMALL = 3, /* a caller buffer is smaller than required */
    MLA_ERR_HIP = 4,                 /* the HIP runtime reported an error */
    MLA_ERR_PLAN_MISMATCH = 5        /* the plan was built for other parameters */
} mla_status;

typedef enum {
    MLA_DTYPE_BF16 = 0,
    MLA_DTYPE_FP32 = 1,
    MLA_DTYPE_FP8_E4M3FN = 2 /* OCP e4m3fn: bias 7, max 448, no infinities */
} mla_dtype;

typedef struct {
    int32_t num_heads;        /* H query heads: 16, 32, 64 or 128 */
    int32_t kv_lora_rank;     /* must be 512 */
    int32_t qk_rope_head_dim; /* must be 64 */
    int32_t page_size;        /* tokens per cache page, >= 1 */
    int32_t kv_dtype;         /* MLA_DTYPE_BF16 or MLA_DTYPE_FP8_E4M3FN */
    int32_t out_dtype;        /* MLA_DTYPE_BF16, or MLA_DTYPE_FP32 for the fp32 mode:
                                 the softmax probabilities and the output are never
                                 rounded to bf16 */
    int32_t num_cus;          /* compute units to balance over; 0 = ask the device */
    int32_t max_splits;       /* cap on KV chunks per query row; 0 = library default,
                                 1 = never split */
    int32_t flags;            /* MLA_DECODE_* bits, 0 for none */
    int32_t max_rows;         /* graph-safe plans: the most query rows any plan will hold
                                 (>= 1); it fixes where the plan's arrays and the partials
                                 sit in the workspace. Ignored otherwise. */
    int32_t suffix_tokens;    /* mla_decode_tree_verify only: the most suffix slots a row
                                 adds after its request's tokens, in [1, 256]; 0 for every
                                 other call */
} mla_decode_params;

/*
 * Graph-safe launches: every grid size and every workspace address of
 * mla_decode (and of the variants below that take a plan) depends on the
 * params only, never on the plan: the plan is laid out for params.max_rows
 * query rows whatever it holds, and the merge kernels read their counts from
 * the plan's device copy. A hipGraph
 * captured around one call therefore stays valid for any later plan built
 * with the same params into the same workspace (by mla_decode_plan on the
 * stream, before the replay), as the graph-replayed decode of the
 * attention-backends page requires: buffers sized for the largest batch,
 * contents changing every step. The decode launch always has all of its
 * workers (those without work exit at once) and the merge launches run
 * even when the plan has no split row, which costs a few microseconds
 * against an ordinary call. Output rows past the plan's query rows are never
 * written (padding rows keep their contents).
 */
#define MLA_DECODE_GRAPH_SAFE 1

/*
 * fp8 score (e4m3fn cache, 128 heads, bf16 output, mla_decode only): the
 * score's contraction runs on the fp8 matrix core, twice the bf16 rate, with
 * the query quantised to e4m3fn. The fp8 cache itself is the FP8 KV cache the
 * SGLang v0.3 MLA page counts among its four decode optimisations; quantising
 * the query too is this library's reading (the pages leave it open): per
 * query row and head, the 576 query values (absorbed no-rope part, then rope
 * part) are scaled by 2^-e, e the smallest integer with amax * 2^-e <= 448
 * (amax their largest magnitude; e = 0 for a head of zeros), which is exact,
 * and rounded to the nearest e4m3fn code, ties to even. The score is then
 * computed from these codes times 2^e. Query values must be finite.
 * mla_decode quantises the query into its workspace with a kernel of its own
 * before the decode launch; the rest of the path (softmax, the P . latent
 * product in bf16, merges) is unchanged. The results differ from the bf16
 * score by the query's rounding (at most 2^-4 of each value) and by the fp8
 * matrix core's internal sums (measured within 2^-12 of the sum of the
 * products' magnitudes).
 */
#define MLA_DECODE_FP8_SCORE 2

/*
 * Shared rows (16 or 32 heads): the query rows of one request (qo_indptr) are
 * planned together, up to 64 / num_heads rows per work item, so that each
 * latent tile the item loads serves all of them: the mixed (q_len > 1)
 * launch the sglang-jax MLA gap page keeps beside the q_len = 1 decode
 * (section 2.4), for MTP and speculative decoding, where a request's draft
 * rows read the same tokens (the PR 49477 analysis, introduction: the prefix
 * that every draft of a request shares). Each row still attends to all of its
 * request's tokens, as without the flag, and the results are the same up to
 * rounding order. The item runs the 64-head kernel with one row's heads per
 * wave (16 heads) or per two waves (32 heads). With 64 or 128 heads one row
 * already fills a work item's accumulators and the flag changes nothing.
 */
#define MLA_DECODE_SHARED_ROWS 4

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(int32_t status);

/*
 * Plan layout. The plan is built on the host and copied verbatim to the start
 * of the device workspace. It is plain data: tests may read it.
 */
#define MLA_PLAN_MAGIC 0x504C4D41u /* "AMLP" */
#define MLA_PLAN_VERSION 7

typedef struct {
    uint32_t magic;
    int32_t version;
    int32_t num_heads, page_size, kv_dtype, out_dtype;
    int32_t batch;          /* requests */
    int32_t num_rows;       /* query rows (qo_indptr[batch]) */
    int32_t num_items;      /* decode work items (a query row and a token range each) */
    int32_t num_merges;     /* query rows whose KV was split into several chunks */
    int32_t num_partials;   /* partial (out, lse) slots written by split chunks */
    int32_t chunk_tokens;   /* per-worker capacity the plan used, in tokens (including
                               a fixed per-item cost counted as tokens) */
    int32_t num_workers;    /* workgroups of the decode launch; worker w processes
                               items [workers[w], workers[w+1]) in order */
    int32_t max_merge_partials; /* most partials any one merged row has (0 without merges) */
    int32_t num_wide_merges; /* the leading merges, those of at least 16 partials */
    int32_t flags;          /* the params' flags the plan was built with */
    int32_t suffix_tokens;  /* the params' suffix_tokens: each row is planned that much longer */
    int32_t tiles_read_once; /* 1: no two items read the same tokens of a request (every
                                request's rows are one item, or one planned unit) */
    int64_t num_page_entries; /* kv_indptr[batch]: entries of kv_indices the batch uses */
    int64_t items_offset;   /* byte offset of mla_work_item[num_items] */
    int64_t merges_offset;  /* byte offset of mla_merge_item[num_merges] */
    int64_t workers_offset; /* byte offset of int32_t workers[num_workers + 1] */
    int64_t plan_bytes;     /* bytes of the plan itself (header + items + merges + workers) */
    int64_t partial_out_offset; /* workspace offset of [num_partials][H][512] partial outputs,
                                   bf16 (fp32 when out_dtype is MLA_DTYPE_FP32) */
    int64_t partial_lse_offset; /* workspace offset of float[num_partials][H] */
    int64_t workspace_bytes;    /* workspace bytes this plan needs */
    int64_t query_codes_offset; /* MLA_DECODE_FP8_SCORE: workspace offset of the quantised
                                   query, uint8 e4m3fn codes [rows][H][576]; else 0 */
    int64_t query_exp_offset;   /* MLA_DECODE_FP8_SCORE: workspace offset of int32 [rows][H],
                                   the exponent e of each row and head; else 0 */
} mla_plan_header;

typedef struct {
    int32_t row;       /* query row n (the first of num_rows consecutive rows) */
    int32_t request;   /* request b */
    int32_t page_base; /* kv_indptr[b]: first entry of b's page list in kv_indices */
    int32_t kv_begin;  /* first token of the chunk */
    int32_t kv_end;    /* one past the last token (the request's length for the last chunk) */
    int32_t partial;   /* -1: write out/lse directly; else the partial slot of row `row`
                          (row + r uses slot partial + r) */
    int32_t head_begin;
    uint32_t flags;    /* MLA_ITEM_* bits */
    int32_t num_rows;  /* query rows row .. row + num_rows - 1 of request b (1 unless
                          MLA_DECODE_SHARED_ROWS) */
    int32_t reserved;
} mla_work_item;

/* The item's chunk ends at its request's planned length (kv_end == L >= 1): the
   item that reads the request's last token, which mla_decode_append writes. */
#define MLA_ITEM_LAST_CHUNK 1u

typedef struct {
    int32_t row;            /* query row n */
    int32_t partial_begin;  /* its chunks are partial slots partial_begin + k * partial_stride, */
    int32_t num_partials;   /*   k < num_partials, in token order */
    int32_t partial_stride; /* 1, or the rows of its shared-rows items */
} mla_merge_item;

/*
 * Upper bounds on the host plan buffer and the device workspace for a batch of
 * up to `batch` requests and `num_rows` query rows with these parameters.
 * Returns MLA_OK, MLA_ERR_INVALID_ARG or MLA_ERR_UNSUPPORTED.
 */
int32_t mla_decode_workspace_size(const mla_decode_params* params, int32_t batch, int32_t num_rows,
                                  size_t* plan_bytes, size_t* workspace_bytes);

/*
 * mla_decode_plan - split-KV chunking and balance across compute units.
 *
 * The CSR description of a paged, ragged batch and the per-batch plan() that
 * picks the split-KV chunking and balances long and short requests across the
 * chip are from the "Paged, ragged batches" paragraph of the SGLang
 * attention-backends page; splitting the keys of one query across workgroups
 * and merging by rescaling is Flash-Decoding, in the FlashAttention paragraph
 * of the same page. A plan is built once per batch and reused by every layer
 * (the PR 49477 analysis, section 1, reuses its metadata across layers).
 *
 *   qo_indptr_h       [batch+1] query rows of each request, or NULL for one row
 *                     per request (plain decode).
 *   kv_indptr_h       [batch+1] offsets of each request's page list in kv_indices.
 *   kv_last_page_len_h [batch] valid tokens in each request's last page, in
 *                     [1, page_size]; NULL means the last page is full. A request
 *                     with no pages has length 0 (its output is 0, lse -inf).
 *   plan_h            caller-owned host buffer (pinned memory is best) of
 *                     plan_h_bytes; receives mla_plan_header + items + merges.
 *   workspace_d       device workspace of workspace_bytes, or NULL to build the
 *                     host plan only. When given, the plan is copied to its
 *                     start with an asynchronous copy on `stream`: plan_h must
 *                     stay unchanged until that copy has completed.
 * The lengths here are upper bounds: mla_decode may clip them further with
 * kv_lens_d. Returns MLA_OK, MLA_ERR_INVALID_ARG (NULL arrays, decreasing
 * indptr, last_page_len out of range), MLA_ERR_UNSUPPORTED,
 * MLA_ERR_WORKSPACE_TOO_SMALL or MLA_ERR_HIP.
 */
int32_t mla_decode_plan(const mla_decode_params* params, int32_t batch, const int32_t* qo_indptr_h,
                        const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                        void* plan_h, size_t plan_h_bytes, void* workspace_d,
                        size_t workspace_bytes, void* stream);

/*
 * mla_decode - absorbed-MLA attention of every query row over its request's
 * paged latent tokens, with split-KV partials merged by log-sum-exp.
 *
 * Formulas: see the top of this header (two-path score and latent reused as
 * value: sglang-jax MLA gap page, sections 2.1 and 2.4; the MLA paragraph of the
 * SGLang attention-backends page; online softmax and split-KV merge: its
 * FlashAttention paragraph). Returns (out, lse) as the fixed-length FA4 path of
 * the PR 49477 analysis, section 4, returns them together.
 *
 *   plan_h, workspace_d  the plan from mla_decode_plan with the same params, and
 *                        the workspace it was copied into.
 *   q_nope_d   bf16 [N, H, 512] absorbed query; element (n, h, d) at
 *              n*q_nope_stride_n + h*q_nope_stride_h + d (strides in elements,
 *              multiples of 8, base 16-byte aligned).
 *   q_rope_d   bf16 [N, H, 64], same conventions. A concatenated [N, H, 576]
 *              query is passed as q_rope_d = q_nope_d + 512 with equal strides.
 *   kv_cache_d [num_pages, page_size, 576] of kv_dtype, rows contiguous
 *              (latent 512, then rope 64); 16-byte aligned.
 *   kv_scale   fp8 dequantisation scale (cache value = code * kv_scale); must be
 *              1 for bf16 caches.
 *   kv_indices_d  int32 page numbers, the CSR column array of the plan's batch;
 *              may be NULL when the batch has no page entries (every request
 *              empty: each row's out is 0 and its lse -inf).
 *   kv_lens_d  int32 [batch] token counts known only on the device, or NULL.
 *              Request b then attends to min(kv_lens_d[b], planned length)
 *              tokens. This is how the tree-verify suffix uses the compacted
 *              table: its lengths come from mla_tree_suffix_compact.
 *   sm_scale   softmax scale applied to the raw scores; finite and > 0.
 *   out_d      [N, H, 512] contiguous, out_dtype.
 *   lse_d      float [N, H] contiguous (natural log), or NULL.
 * Reads: for each request, the cache rows of its tokens below its length,
 * at the pages its kv_indices entries name, and nothing else of the cache.
 * The library takes no pool size: it does not check those page numbers
 * against the pool, and an entry outside it is an out-of-bounds device read.
 * Callers that cannot vouch for their page tables check them on the host with
 * mla_decode_validate_batch before the call. Returns MLA_OK, MLA_ERR_INVALID_ARG,
 * MLA_ERR_UNSUPPORTED, MLA_ERR_PLAN_MISMATCH, MLA_ERR_WORKSPACE_TOO_SMALL or
 * MLA_ERR_HIP.
 */
int32_t mla_decode(const mla_decode_params* params, const void* plan_h, const void* workspace_d,
                   size_t workspace_bytes, const void* q_nope_d, int64_t q_nope_stride_n,
                   int64_t q_nope_stride_h, const void* q_rope_d, int64_t q_rope_stride_n,
                   int64_t q_rope_stride_h, const void* kv_cache_d, float kv_scale,
                   const int32_t* kv_indices_d, const int32_t* kv_lens_d, float sm_scale,
                   void* out_d, float* lse_d, void* stream);

/*
 * mla_decode_noalloc - mla_decode without a workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The plan (built by mla_decode_plan
 * with workspace_d = NULL) is copied by this call into a scratch array the
 * library keeps in device memory (64 MiB per GPU, held until the process
 * ends), which also holds the split-KV partials; the call allocates nothing.
 * plan_h must stay unchanged until that asynchronous copy has run.
 *
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * there: calls that overlap on one GPU (different streams, or different
 * threads without ordering) race and give wrong results. Everything the
 * kernels need zeroed comes with the plan copy of each call.
 *
 * Arguments and results as for mla_decode (without workspace_d and
 * workspace_bytes). Returns those of mla_decode, and
 * MLA_ERR_WORKSPACE_TOO_SMALL when the plan needs more than the 64 MiB
 * scratch (mla_decode_workspace_size reports the bytes; at 128 heads a
 * bf16 partial is 128 KiB, so about 500 split-KV pieces fit).
 */
int32_t mla_decode_noalloc(const mla_decode_params* params, const void* plan_h,
                           const void* q_nope_d, int64_t q_nope_stride_n, int64_t q_nope_stride_h,
                           const void* q_rope_d, int64_t q_rope_stride_n, int64_t q_rope_stride_h,
                           const void* kv_cache_d, float kv_scale, const int32_t* kv_indices_d,
                           const int32_t* kv_lens_d, float sm_scale, void* out_d, float* lse_d,
                           void* stream);

/*
 * mla_decode_append - mla_decode with the new token's cache row written in the
 * same launch (the fused KV-cache update of the tpu-inference V2 MLA kernel,
 * sglang-jax MLA gap page, section 2.4; the nope and rope parts are written
 * separately as the MLA token pool's set_mla_kv_buffer does, section 3.1).
 *
 * Each request b has exactly one query row n (qo_indptr was NULL or the
 * identity) and a planned length L_b >= 1 that already counts the new token.
 * Before any of its tokens is read, the row of token L_b - 1 (page
 * kv_indices[kv_indptr[b] + (L_b-1)/page_size], in-page row (L_b-1) % page_size)
 * becomes
 *   latent = c_new[n, 0:512], rope = k_pe_new[n, 0:64]        (bf16 cache), or
 *   code(v) = e4m3fn_rne(clamp(v / kv_scale, -448, 448))      (fp8 cache),
 * with v / kv_scale an IEEE fp32 division and e4m3fn_rne the round-to-nearest-
 * even OCP e4m3fn encoding. The attention then runs as mla_decode over all
 * L_b tokens, the new one read back from the cache as stored. The result is
 * that of writing the row first and calling mla_decode, without a separate
 * launch or a read of the row through another kernel.
 *
 *   kv_cache_d   as for mla_decode, but written: only the L_b - 1 row of each
 *                request changes.
 *   c_new_d      bf16 [N, 512], row n at n*c_new_stride (elements, multiple of 8);
 *                16-byte aligned. Finite values.
 *   k_pe_new_d   bf16 [N, 64], row n at n*k_pe_new_stride, same conventions
 *                (a concatenated [N, 576] row is c_new_d with k_pe_new_d = c_new_d + 512).
 *   kv_lens_d    not taken: the planned lengths are the lengths.
 * Other arguments as for mla_decode. Returns those of mla_decode, and
 * MLA_ERR_INVALID_ARG when a request has no token or more than one query row.
 */
int32_t mla_decode_append(const mla_decode_params* params, const void* plan_h,
                          const void* workspace_d, size_t workspace_bytes, const void* q_nope_d,
                          int64_t q_nope_stride_n, int64_t q_nope_stride_h, const void* q_rope_d,
                          int64_t q_rope_stride_n, int64_t q_rope_stride_h, void* kv_cache_d,
                          float kv_scale, const int32_t* kv_indices_d, const void* c_new_d,
                          int64_t c_new_stride, const void* k_pe_new_d, int64_t k_pe_new_stride,
                          float sm_scale, void* out_d, float* lse_d, void* stream);

/*
 * mla_decode_suffix_merge - mla_decode whose result is merged by LSE with a
 * given state over other tokens, in the same call: the fused suffix-attention
 * + merge of the tree-verify cascade (PR 49477 analysis, section 3), where the
 * suffix attention over the compacted draft slots meets the prefix state.
 * With (v_p, s_p) the given state and (v, s) this call's attention,
 *   lse = ln(e^{s_p} + e^{s}),  out = e^{s_p - lse} v_p + e^{s - lse} v,
 * exactly mla_merge_states(prefix, mla_decode(...)) up to rounding; an empty
 * side drops out, two empty sides give out 0 and lse -inf. Unsplit rows merge
 * in the decode kernel's output stage and split rows in the split-KV merge, so
 * this call's own (out, lse) never goes through memory.
 *
 *   prefix_out_d  [N, H, 512] in out_dtype, contiguous, 16-byte aligned.
 *   prefix_lse_d  float [N, H] contiguous (natural log).
 *   out_d, lse_d  as for mla_decode; each either the same memory as the
 *                 prefix array of its kind (an in-place merge) or disjoint
 *                 from it.
 * Other arguments, kv_lens_d included, as for mla_decode. Returns those of
 * mla_decode.
 */
int32_t mla_decode_suffix_merge(const mla_decode_params* params, const void* plan_h,
                                const void* workspace_d, size_t workspace_bytes,
                                const void* q_nope_d, int64_t q_nope_stride_n,
                                int64_t q_nope_stride_h, const void* q_rope_d,
                                int64_t q_rope_stride_n, int64_t q_rope_stride_h,
                                const void* kv_cache_d, float kv_scale, const int32_t* kv_indices_d,
                                const int32_t* kv_lens_d, float sm_scale, const void* prefix_out_d,
                                const float* prefix_lse_d, void* out_d, float* lse_d, void* stream);

/*
 * mla_decode_tree_verify - the tree-verify attention of the PR 49477 analysis
 * in one pass: every draft row attends to its request's prefix and, in the same
 * softmax, to its visible draft slots, instead of a prefix pass, a suffix pass
 * over the compacted table (section 2) and an LSE merge of the two (section 3).
 * The result is the cascade's: attention over the union of the two token sets.
 *
 * For query row n of request b (rows by qo_indptr, as planned): the request's
 * L_b planned tokens through kv_indices_d, then the pool rows
 * suffix_table_d[n*suffix_stride + j] for j < min(suffix_lens_d[n], S), with
 * S = params.suffix_tokens. These are the page_table and cache_seqlens that
 * mla_tree_suffix_compact writes (its table_stride as suffix_stride, S the
 * max_tree_depth of its truncation); rows with suffix_lens_d[n] = 0 attend to
 * the prefix only.
 *
 * Requirements: params.num_heads = 128, params.page_size = 1 (suffix entries
 * are token slots, that is pool rows), params.suffix_tokens = S in [1, 256],
 * and a plan built with those params (each row is planned S tokens longer, its
 * last chunk holding all of them). suffix_stride >= S. Every suffix entry read
 * is a row of the pool. Other arguments as for mla_decode (no kv_lens_d).
 * Returns those of mla_decode; MLA_ERR_INVALID_ARG for a missing table or
 * lengths, or when a plan with suffix_tokens > 0 reaches any other call.
 */
int32_t mla_decode_tree_verify(const mla_decode_params* params, const void* plan_h,
                               const void* workspace_d, size_t workspace_bytes,
                               const void* q_nope_d, int64_t q_nope_stride_n,
                               int64_t q_nope_stride_h, const void* q_rope_d,
                               int64_t q_rope_stride_n, int64_t q_rope_stride_h,
                               const void* kv_cache_d, float kv_scale, const int32_t* kv_indices_d,
                               const int32_t* suffix_table_d, int64_t suffix_stride,
                               const int32_t* suffix_lens_d, float sm_scale, void* out_d,
                               float* lse_d, void* stream);

/*
 * mla_merge_states - merge two attention states over disjoint token sets:
 *   s = ln(e^{s_a} + e^{s_b}),  v = e^{s_a - s} v_a + e^{s_b - s} v_b.
 * This is the LSE merge of the prefix and suffix results in the cascade of the
 * PR 49477 analysis (introduction), and the Flash-Decoding rescaling of the
 * attention-backends page. A state with s = -inf (no tokens) drops out; two
 * empty states give v = 0, s = -inf.
 *
 *   v_a_d, v_b_d, v_out_d  [num_rows, head_dim] of v_dtype (BF16 or FP32, all
 *                          three the same), rows contiguous, 16-byte aligned.
 *   s_a_d, s_b_d, s_out_d  float [num_rows], natural-log LSE.
 *   head_dim               multiple of 8, at most 4096.
 * v_out_d may alias v_a_d or v_b_d (and s_out_d s_a_d or s_b_d).
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int32_t mla_merge_states(const void* v_a_d, const float* s_a_d, const void* v_b_d,
                         const float* s_b_d, void* v_out_d, float* s_out_d, int64_t num_rows,
                         int32_t head_dim, int32_t v_dtype, void* stream);

/*
 * mla_tree_suffix_compact - suffix page table of tree-verify attention by a
 * scan-based stable compaction, in one launch (PR 49477 analysis, section 1).
 *
 * For query row r < num_actual_rows, request req = r / width:
 *   valid[c] = tree_mask_d[r*mask_stride + c] != 0          (c < width)
 *   rank[c]  = inclusive prefix sum of valid; count = sum of valid
 *   dest[c]  = valid[c] ? rank[c]-1 : count + c - rank[c]
 *   page_table_d[r*table_stride + dest[c]] =
 *            req_to_token_d[req*req_stride + prefix_lens_d[req] + c]
 *   cache_seqlens_d[r] = count
 * i.e. visible draft slots first and then the hidden ones, each group in its
 * original order. Rows num_actual_rows <= r < num_rows are graph padding: no
 * mask is read, the table row is zeroed and the length is 0. Because the
 * visible slots come first, attending to the first cache_seqlens_d[r] entries
 * of each row is the truncation to max_tree_depth of section 2 (pass
 * cache_seqlens_d as kv_lens_d to mla_decode).
 *   tree_mask_d  uint8 [num_actual_rows, mask_stride], mask_stride >= width
 *   req_to_token_d int32 [*, req_stride]; prefix_lens_d int32 [num_actual_rows/width rounded up]
 *   page_table_d int32 [num_rows, table_stride], table_stride >= width
 *   width in [1, 1024]
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int32_t mla_tree_suffix_compact(const uint8_t* tree_mask_d, int64_t mask_stride,
                                const int32_t* req_to_token_d, int64_t req_stride,
                                const int32_t* prefix_lens_d, int32_t width, int32_t num_rows,
                                int32_t num_actual_rows, int32_t* page_table_d,
                                int64_t table_stride, int32_t* cache_seqlens_d, void* stream);

/*
 * mla_absorb_query - the query side of weight absorption: fold W_UK into the
 * no-rope query so that scores are taken directly against the cached latent
 * (SGLang v0.3 MLA page, weight absorption; sglang-jax MLA gap page, sections
 * 2.1-2.2):
 *   q_abs[n,h,a] = sum_d q[n,h,d] * W_UK[a,h,d]        (a < 512, d < head_dim)
 * where the per-head key is k_nope[t,h,d] = sum_a c[t,a] * W_UK[a,h,d], so
 * q_abs[n,h,:] . c_t = q[n,h,:] . k_nope[t,h,:]. bf16 in and out, fp32
 * accumulation, one rounding to bf16 per output.
 *
 *   q_d       bf16 [N, H, head_dim]; element (n, h, d) at n*q_stride_n + h*q_stride_h + d.
 *   w_uk_d    bf16 W_UK; element (a, h, d) at a*w_uk_stride_a + h*w_uk_stride_h + d
 *             (d contiguous: [512, H, head_dim] or [H, 512, head_dim] both fit).
 *   q_abs_d   bf16 [N, H, 512]; element (n, h, a) at n*q_abs_stride_n + h*q_abs_stride_h + a.
 *             Writing into a concatenated [N, H, 576] decode query (strides
 *             H*576 and 576) leaves its rope part untouched.
 *   head_dim  must be 128. num_heads in [1, 65535], num_rows in [0, 2097120].
 * All strides in elements, non-negative multiples of 8; bases 16-byte aligned.
 * q_abs_d must not overlap q_d or w_uk_d. Returns MLA_OK, MLA_ERR_INVALID_ARG,
 * MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int32_t mla_absorb_query(const void* q_d, int64_t q_stride_n, int64_t q_stride_h, const void* w_uk_d,
                         int64_t w_uk_stride_a, int64_t w_uk_stride_h, void* q_abs_d,
                         int64_t q_abs_stride_n, int64_t q_abs_stride_h, int32_t num_rows,
                         int32_t num_heads, int32_t head_dim, void* stream);

/*
 * mla_project_output - the output side of weight absorption: map the per-head
 * attention result over latents (what mla_decode writes) to the value head
 * dimension with W_UV (SGLang v0.3 MLA page, weight absorption; sglang-jax MLA
 * gap page, section 2.2):
 *   o[n,h,d] = sum_a x[n,h,a] * W_UV[a,h,d]             (a < 512, d < head_dim)
 * the same result as attending over the decompressed values
 * v[t,h,d] = sum_a c[t,a] * W_UV[a,h,d]. bf16 in and out, fp32 accumulation.
 *
 *   x_d       bf16 [N, H, 512]; element (n, h, a) at n*x_stride_n + h*x_stride_h + a.
 *   w_uv_d    bf16 W_UV; element (a, h, d) at h*w_uv_stride_h + d*w_uv_stride_d + a
 *             (a contiguous: the value rows of a kv_b_proj weight stored
 *             [H*(dn+dv), 512] fit with stride_h (dn+dv)*512, stride_d 512, base
 *             advanced by dn*512).
 *   o_d       bf16 [N, H, head_dim]; element (n, h, d) at n*o_stride_n + h*o_stride_h + d.
 *   head_dim  must be 128. num_heads in [1, 65535], num_rows in [0, 2097120].
 * All strides in elements, non-negative multiples of 8; bases 16-byte aligned.
 * o_d must not overlap x_d or w_uv_d. Returns MLA_OK, MLA_ERR_INVALID_ARG,
 * MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int32_t mla_project_output(const void* x_d, int64_t x_stride_n, int64_t x_stride_h, const void* w_uv_d,
                           int64_t w_uv_stride_h, int64_t w_uv_stride_d, void* o_d,
                           int64_t o_stride_n, int64_t o_stride_h, int32_t num_rows,
                           int32_t num_heads, int32_t head_dim, void* stream);

/*
 * Host checks of a batch's index arrays against the pool, for callers that
 * cannot vouch for them (the decode entry points take no pool size and read
 * whatever rows the entries name). They read host copies only, enqueue
 * nothing and need no device. Graph padding in the PR 49477 analysis
 * (section 1) pins padded rows to offset 0 for exactly this reason: an index
 * past the pool is an out-of-bounds read on the device.
 *
 * mla_decode_validate_batch: kv_indptr_h [batch+1] (and qo_indptr_h, when not
 * NULL) start at 0 and never decrease; every entry kv_indices_h[e],
 * e < kv_indptr_h[batch], is a page of the pool, 0 <= page < num_pool_pages;
 * kv_last_page_len_h (when not NULL) is in [1, page_size] for every request
 * with pages.
 *
 * mla_tree_validate_inputs: the inputs of mla_tree_suffix_compact. For every
 * request r < num_requests, 0 <= prefix_lens_h[r] and prefix_lens_h[r] + width
 * <= req_stride (the compaction reads req_to_token at columns
 * [prefix_len, prefix_len + width)), and each of those draft slots is a pool
 * row, 0 <= slot < num_pool_rows. req_to_token_h [num_requests, req_stride].
 *
 * mla_tree_validate_suffix: what mla_decode_tree_verify reads of the compacted
 * table. For every row n < num_rows, suffix_lens_h[n] >= 0 and the entries
 * suffix_table_h[n*suffix_stride + j], j < min(suffix_lens_h[n],
 * suffix_tokens), are pool rows, 0 <= slot < num_pool_rows.
 *
 * Each returns MLA_OK, or MLA_ERR_INVALID_ARG for malformed arguments or the
 * first entry out of range; *bad_entry (when not NULL) receives that entry's
 * index in its array, or -1 when no single entry is at fault.
 */
int32_t mla_decode_validate_batch(int32_t page_size, int32_t batch, const int32_t* qo_indptr_h,
                                  const int32_t* kv_indptr_h, const int32_t* kv_indices_h,
                                  const int32_t* kv_last_page_len_h, int64_t num_pool_pages,
                                  int64_t* bad_entry);
int32_t mla_tree_validate_inputs(const int32_t* req_to_token_h, int64_t req_stride,
                                 int32_t num_requests, const int32_t* prefix_lens_h, int32_t width,
                                 int64_t num_pool_rows, int64_t* bad_entry);
int32_t mla_tree_validate_suffix(const int32_t* suffix_table_h, int64_t suffix_stride,
                                 const int32_t* suffix_lens_h, int32_t num_rows,
                                 int32_t suffix_tokens, int64_t num_pool_rows, int64_t* bad_entry);

/*
 * Name of the decode kernel instantiation these parameters select (static
 * storage), e.g. "mla_decode<hw32,hs4,kv_bf16,out_bf16>"; NULL if unsupported.
 * Tests use it to prove which branch ran.
 */
const char* mla_decode_variant(const mla_decode_params* params);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
