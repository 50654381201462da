// C-ABI entry points of the MLA decode library: argument validation on the
// host, then launches on the caller's stream. See include/mla_decode.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "mla_decode.h"
#include "mla_internal.h"

using namespace mla;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_cu_mutex;
int g_cu_count[kMaxDevices] = {0};

// Compute units of the current device (cached per device).
int32_t device_cus(int32_t requested, int32_t* out) {
    if (requested > 0) {
        *out = requested;
        return MLA_OK;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return MLA_ERR_HIP;
        g_cu_count[dev] = n;
    }
    *out = g_cu_count[dev];
    return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

const char* mla_status_string(int32_t status) {
    switch (status) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
        case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
        case MLA_ERR_HIP: return "MLA_ERR_HIP";
        case MLA_ERR_PLAN_MISMATCH: return "MLA_ERR_PLAN_MISMATCH";
        default: return "MLA_ERR_UNKNOWN";
    }
}

const char* mla_decode_variant(const mla_decode_params* params) { return variant_name(params); }

int32_t mla_decode_workspace_size(const mla_decode_params* params, int32_t batch, int32_t num_rows,
                                  size_t* plan_bytes, size_t* workspace_bytes) {
    if (!params || (!plan_bytes && !workspace_bytes)) return MLA_ERR_INVALID_ARG;
    Variant v;
    if (!select_variant(params, &v)) return MLA_ERR_UNSUPPORTED;
    int32_t cus = 0;
    const int32_t st = device_cus(params->num_cus, &cus);
    if (st != MLA_OK) return st;
    return plan_bounds(params, cus, batch, num_rows, plan_bytes, workspace_bytes);
}

int32_t mla_decode_plan(const mla_decode_params* params, int32_t batch, const int32_t* qo_indptr_h,
                        const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                        void* plan_h, size_t plan_h_bytes, void* workspace_d,
                        size_t workspace_bytes, void* stream) {
    if (!params || !kv_indptr_h || !plan_h || batch < 0) return MLA_ERR_INVALID_ARG;
    Variant v;
    if (!select_variant(params, &v)) return MLA_ERR_UNSUPPORTED;
    int32_t cus = 0;
    int32_t st = device_cus(params->num_cus, &cus);
    if (st != MLA_OK) return st;
    st = plan_build(params, cus, batch, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, plan_h,
                    plan_h_bytes);
    if (st != MLA_OK) return st;
    const mla_plan_header* h = static_cast<const mla_plan_header*>(plan_h);
    if (workspace_d) {
        if ((size_t)h->workspace_bytes > workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
        if (hipMemcpyAsync(workspace_d, plan_h, (size_t)h->plan_bytes, hipMemcpyHostToDevice,
                           (hipStream_t)stream) != hipSuccess)
            return MLA_ERR_HIP;
    }
    return MLA_OK;
}

}  // extern "C"

namespace {

// The new-token inputs of mla_decode_append.
struct AppendIn {
    const void* c_new;
    int64_t c_new_stride;
    const void* k_pe_new;
    int64_t k_pe_new_stride;
};

// The prefix state of mla_decode_suffix_merge.
struct PrefixIn {
    const void* out;
    const float* lse;
};

// The suffix slots of mla_decode_tree_verify.
struct TreeIn {
    const int32_t* table;
    int64_t stride;
    const int32_t* lens;
};

// Two byte ranges that are either the same or disjoint.
bool same_or_disjoint(const void* x, const void* y, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a == b || a + bytes <= b || b + bytes <= a;
}

// Every request has exactly one query row and a last-chunk item (length >= 1).
bool append_batch_ok(const mla_plan_header* h, const void* plan_h) {
    if (h->num_rows != h->batch) return false;
    const mla_work_item* items =
        reinterpret_cast<const mla_work_item*>(static_cast<const char*>(plan_h) + h->items_offset);
    std::vector<char> seen((size_t)h->batch, 0);
    int32_t n = 0;
    for (int32_t i = 0; i < h->num_items; ++i) {
        if (!(items[i].flags & MLA_ITEM_LAST_CHUNK)) continue;
        const int32_t b = items[i].request;
        if (b < 0 || b >= h->batch || seen[(size_t)b]) return false;
        seen[(size_t)b] = 1;
        ++n;
    }
    return n == h->batch;
}

int32_t decode_impl(const mla_decode_params* params, const void* plan_h, const void* workspace_d,
                    size_t workspace_bytes, const void* q_nope_d, int64_t q_nope_stride_n,
                    int64_t q_nope_stride_h, const void* q_rope_d, int64_t q_rope_stride_n,
                    int64_t q_rope_stride_h, const void* kv_cache_d, float kv_scale,
                    const int32_t* kv_indices_d, const int32_t* kv_lens_d, const AppendIn* app,
                    const PrefixIn* pre, const TreeIn* tree, float sm_scale, void* out_d, float* lse_d,
                    void* stream, bool copy_plan = false) {
    if (!params || !plan_h || !workspace_d) return MLA_ERR_INVALID_ARG;
    Variant v;
    if (!select_variant(params, &v)) return MLA_ERR_UNSUPPORTED;
    const mla_plan_header* h = static_cast<const mla_plan_header*>(plan_h);
    if (h->magic != MLA_PLAN_MAGIC || h->version != MLA_PLAN_VERSION) return MLA_ERR_INVALID_ARG;
    if (h->num_heads != params->num_heads || h->page_size != params->page_size ||
        h->kv_dtype != params->kv_dtype || h->out_dtype != params->out_dtype ||
        h->flags != params->flags || h->suffix_tokens != params->suffix_tokens)
        return MLA_ERR_PLAN_MISMATCH;
    // suffix_tokens plans are for the tree-verify call, and it needs one.
    if ((params->suffix_tokens > 0) != (tree != nullptr)) return MLA_ERR_INVALID_ARG;
    if (tree && (!tree->table || !tree->lens || tree->stride < params->suffix_tokens))
        return MLA_ERR_INVALID_ARG;
    if ((size_t)h->workspace_bytes > workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
    // A graph-safe call launches whatever this plan holds: a later plan may not be empty.
    const bool graph = (params->flags & MLA_DECODE_GRAPH_SAFE) != 0;
    if (h->num_items == 0 && !graph) return MLA_OK;
    // A batch of empty requests has no page entries, and its page array may be NULL.
    if (!q_nope_d || !q_rope_d || !kv_cache_d || (!kv_indices_d && h->num_page_entries > 0) || !out_d)
        return MLA_ERR_INVALID_ARG;
    if (!aligned16(q_nope_d) || !aligned16(q_rope_d) || !aligned16(kv_cache_d) || !aligned16(out_d) ||
        !aligned16(workspace_d))
        return MLA_ERR_INVALID_ARG;
    if (q_nope_stride_n < 0 || q_nope_stride_h < 0 || q_rope_stride_n < 0 || q_rope_stride_h < 0 ||
        (q_nope_stride_n | q_nope_stride_h | q_rope_stride_n | q_rope_stride_h) % 8 != 0)
        return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale) || sm_scale <= 0.f || !std::isfinite(kv_scale) || kv_scale <= 0.f)
        return MLA_ERR_INVALID_ARG;
    if (params->kv_dtype == MLA_DTYPE_BF16 && kv_scale != 1.f) return MLA_ERR_INVALID_ARG;
    // The fp8 score is a variant of the plain decode only.
    const bool qf8 = (params->flags & MLA_DECODE_FP8_SCORE) != 0;
    if (qf8 && (app || pre || tree)) return MLA_ERR_UNSUPPORTED;
    if (app) {
        if (!app->c_new || !app->k_pe_new || !aligned16(app->c_new) || !aligned16(app->k_pe_new) ||
            app->c_new_stride < 0 || app->k_pe_new_stride < 0 ||
            (app->c_new_stride | app->k_pe_new_stride) % 8 != 0)
            return MLA_ERR_INVALID_ARG;
        if (!append_batch_ok(h, plan_h)) return MLA_ERR_INVALID_ARG;
    }
    if (pre) {
        if (!pre->out || !pre->lse || !aligned16(pre->out) || (reinterpret_cast<uintptr_t>(pre->lse) & 3))
            return MLA_ERR_INVALID_ARG;
        const size_t elems = (size_t)h->num_rows * (size_t)params->num_heads;
        const size_t ebytes = params->out_dtype == MLA_DTYPE_FP32 ? 4 : 2;
        if (!same_or_disjoint(out_d, pre->out, elems * kLatent * ebytes)) return MLA_ERR_INVALID_ARG;
        if (lse_d && !same_or_disjoint(lse_d, pre->lse, elems * 4)) return MLA_ERR_INVALID_ARG;
    }

    const char* ws = static_cast<const char*>(workspace_d);
    DecodeArgs a{};
    a.items = reinterpret_cast<const mla_work_item*>(ws + h->items_offset);
    a.workers = reinterpret_cast<const int32_t*>(ws + h->workers_offset);
    a.q_nope = static_cast<const uint16_t*>(q_nope_d);
    a.qn_sn = q_nope_stride_n;
    a.qn_sh = q_nope_stride_h;
    a.q_rope = static_cast<const uint16_t*>(q_rope_d);
    a.qr_sn = q_rope_stride_n;
    a.qr_sh = q_rope_stride_h;
    a.cache = static_cast<const uint8_t*>(kv_cache_d);
    a.kv_indices = kv_indices_d;
    a.kv_lens = kv_lens_d;
    a.out = out_d;
    a.lse = lse_d;
    a.part_out = const_cast<char*>(ws) + h->partial_out_offset;
    a.part_lse = reinterpret_cast<float*>(const_cast<char*>(ws) + h->partial_lse_offset);
    a.num_heads = params->num_heads;
    a.page_size = params->page_size;
    a.page_shift = -1;
    for (int b = 0; b < 31; ++b)
        if (params->page_size == (1 << b)) a.page_shift = b;
    a.scale_log2 = (float)((double)sm_scale * (double)kv_scale * 1.4426950408889634);
    a.out_scale = kv_scale;
    // Tiles read once per launch (one planned unit of rows per request) stream past the
    // caches, which then keep the queries the pieces of a row share and the
    // partials the merge reads back (A/B on one box: V3 133.1-133.6 -> 130.0-
    // 130.5 us, V2-Lite 41.4 -> 37.9 us per call). Rows that share a request's
    // tiles (qo_indptr, tree verify) keep the default policy, under which L2
    // serves the repeats (the hint cost the tree-verify pass 531 -> 544 us),
    // and so do fp8 tiles (rows of 576 bytes straddle cache lines; skewed fp8
    // 67.3 -> 70.2 us with it). A graph-safe launch keeps the choice of the
    // plan it was captured with.
    a.stream_tiles = params->kv_dtype == MLA_DTYPE_BF16 && h->tiles_read_once && !tree;
    if (app) {
        a.c_new = static_cast<const uint16_t*>(app->c_new);
        a.c_new_sn = app->c_new_stride;
        a.k_pe_new = static_cast<const uint16_t*>(app->k_pe_new);
        a.k_pe_new_sn = app->k_pe_new_stride;
        a.cache_w = static_cast<uint8_t*>(const_cast<void*>(kv_cache_d));
        a.kv_scale = kv_scale;
    }
    if (pre) {
        a.prefix_out = pre->out;
        a.prefix_lse = pre->lse;
    }
    if (tree) {
        a.sfx_table = tree->table;
        a.sfx_stride = tree->stride;
        a.sfx_lens = tree->lens;
        a.sfx_max = params->suffix_tokens;
    }
    // mla_decode_noalloc: the plan goes to the library's scratch first.
    if (copy_plan && hipMemcpyAsync(const_cast<void*>(workspace_d), plan_h, (size_t)h->plan_bytes,
                                    hipMemcpyHostToDevice, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_HIP;
    if (qf8) {
        QuantQueryArgs q{};
        q.q_nope = a.q_nope;
        q.qn_sn = q_nope_stride_n;
        q.qn_sh = q_nope_stride_h;
        q.q_rope = a.q_rope;
        q.qr_sn = q_rope_stride_n;
        q.qr_sh = q_rope_stride_h;
        q.num_heads = params->num_heads;
        q.dev_num_rows = &reinterpret_cast<const mla_plan_header*>(ws)->num_rows;
        q.codes = reinterpret_cast<uint8_t*>(const_cast<char*>(ws) + h->query_codes_offset);
        q.exps = reinterpret_cast<int32_t*>(const_cast<char*>(ws) + h->query_exp_offset);
        // Graph-safe: a grid for max_rows rows, whatever this plan holds.
        const int rows = graph ? params->max_rows : h->num_rows;
        if (rows > 0 && launch_quantize_query(q, rows, stream) != 0) return MLA_ERR_HIP;
        a.q8 = q.codes;
        a.q8_exp = q.exps;
    }
    int err = launch_decode(v, params->kv_dtype, params->out_dtype, a, h->num_workers, stream);
    if (err != 0) return MLA_ERR_HIP;
    if (h->num_merges > 0 || graph) {
        MergePartialsArgs m{};
        m.merges = reinterpret_cast<const mla_merge_item*>(ws + h->merges_offset);
        m.part_out = a.part_out;
        m.part_lse = a.part_lse;
        m.out = out_d;
        m.lse = lse_d;
        m.num_heads = params->num_heads;
        m.prefix_out = a.prefix_out;
        m.prefix_lse = a.prefix_lse;
        // Merges come most partials first (planner); the leading ones are wide.
        int num_merges = h->num_merges, num_wide = h->num_wide_merges;
        if (graph) {
            // Fixed grids that bound any plan of these params: every split row
            // crosses at least one of the G - 1 worker boundaries, a wide one at
            // least 15, and no boundary is crossed twice.
            const mla_plan_header* hd = reinterpret_cast<const mla_plan_header*>(ws);
            m.dev_num_merges = &hd->num_merges;
            m.dev_num_wide = &hd->num_wide_merges;
            // With shared rows each split unit holds up to rows_per_item rows.
            const int g = h->num_workers;
            num_merges = std::max(1, g - 1) * v.rows_per_item;
            num_wide = std::max(1, (g - 1 + kWideMergePartials - 2) / (kWideMergePartials - 1)) * v.rows_per_item;
        }
        err = launch_merge_partials(params->out_dtype, m, num_merges, num_wide, stream);
        if (err != 0) return MLA_ERR_HIP;
    }
    return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_decode(const mla_decode_params* params, const void* plan_h, const void* workspace_d,
                   size_t workspace_bytes, const void* q_nope_d, int64_t q_nope_stride_n,
                   int64_t q_nope_stride_h, const void* q_rope_d, int64_t q_rope_stride_n,
                   int64_t q_rope_stride_h, const void* kv_cache_d, float kv_scale,
                   const int32_t* kv_indices_d, const int32_t* kv_lens_d, float sm_scale,
                   void* out_d, float* lse_d, void* stream) {
    return decode_impl(params, plan_h, workspace_d, workspace_bytes, q_nope_d, q_nope_stride_n,
                       q_nope_stride_h, q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d,
                       kv_scale, kv_indices_d, kv_lens_d, nullptr, nullptr, nullptr, sm_scale, out_d,
                       lse_d, stream);
}

int32_t mla_decode_noalloc(const mla_decode_params* params, const void* plan_h,
                           const void* q_nope_d, int64_t q_nope_stride_n, int64_t q_nope_stride_h,
                           const void* q_rope_d, int64_t q_rope_stride_n, int64_t q_rope_stride_h,
                           const void* kv_cache_d, float kv_scale, const int32_t* kv_indices_d,
                           const int32_t* kv_lens_d, float sm_scale, void* out_d, float* lse_d,
                           void* stream) {
    if (!params || !plan_h) return MLA_ERR_INVALID_ARG;
    const mla_plan_header* h = static_cast<const mla_plan_header*>(plan_h);
    if (h->magic != MLA_PLAN_MAGIC || h->version != MLA_PLAN_VERSION) return MLA_ERR_INVALID_ARG;
    // The plan and everything it places in the workspace must fit the scratch.
    if (h->workspace_bytes < h->plan_bytes || (size_t)h->workspace_bytes > kNoAllocScratchBytes)
        return MLA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const int32_t st = noalloc_scratch(&ws);
    if (st != MLA_OK) return st;
    // decode_impl copies the plan to the start of the scratch (as mla_decode_plan
    // puts it at the start of a workspace) after its argument checks.
    return decode_impl(params, plan_h, ws, kNoAllocScratchBytes, q_nope_d, q_nope_stride_n, q_nope_stride_h,
                       q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d, kv_scale, kv_indices_d,
                       kv_lens_d, nullptr, nullptr, nullptr, sm_scale, out_d, lse_d, stream,
                       /*copy_plan=*/true);
}

int32_t mla_decode_tree_verify(const mla_decode_params* params, const void* plan_h,
                               const void* workspace_d, size_t workspace_bytes,
                               const void* q_nope_d, int64_t q_nope_stride_n,
                               int64_t q_nope_stride_h, const void* q_rope_d,
                               int64_t q_rope_stride_n, int64_t q_rope_stride_h,
                               const void* kv_cache_d, float kv_scale, const int32_t* kv_indices_d,
                               const int32_t* suffix_table_d, int64_t suffix_stride,
                               const int32_t* suffix_lens_d, float sm_scale, void* out_d,
                               float* lse_d, void* stream) {
    const TreeIn tree{suffix_table_d, suffix_stride, suffix_lens_d};
    return decode_impl(params, plan_h, workspace_d, workspace_bytes, q_nope_d, q_nope_stride_n,
                       q_nope_stride_h, q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d,
                       kv_scale, kv_indices_d, nullptr, nullptr, nullptr, &tree, sm_scale, out_d,
                       lse_d, stream);
}

int32_t mla_decode_suffix_merge(const mla_decode_params* params, const void* plan_h,
                                const void* workspace_d, size_t workspace_bytes,
                                const void* q_nope_d, int64_t q_nope_stride_n,
                                int64_t q_nope_stride_h, const void* q_rope_d,
                                int64_t q_rope_stride_n, int64_t q_rope_stride_h,
                                const void* kv_cache_d, float kv_scale, const int32_t* kv_indices_d,
                                const int32_t* kv_lens_d, float sm_scale, const void* prefix_out_d,
                                const float* prefix_lse_d, void* out_d, float* lse_d, void* stream) {
    const PrefixIn pre{prefix_out_d, prefix_lse_d};
    return decode_impl(params, plan_h, workspace_d, workspace_bytes, q_nope_d, q_nope_stride_n,
                       q_nope_stride_h, q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d,
                       kv_scale, kv_indices_d, kv_lens_d, nullptr, &pre, nullptr, sm_scale, out_d,
                       lse_d, stream);
}

int32_t mla_decode_append(const mla_decode_params* params, const void* plan_h,
                          const void* workspace_d, size_t workspace_bytes, const void* q_nope_d,
                          int64_t q_nope_stride_n, int64_t q_nope_stride_h, const void* q_rope_d,
                          int64_t q_rope_stride_n, int64_t q_rope_stride_h, void* kv_cache_d,
                          float kv_scale, const int32_t* kv_indices_d, const void* c_new_d,
                          int64_t c_new_stride, const void* k_pe_new_d, int64_t k_pe_new_stride,
                          float sm_scale, void* out_d, float* lse_d, void* stream) {
    const AppendIn app{c_new_d, c_new_stride, k_pe_new_d, k_pe_new_stride};
    return decode_impl(params, plan_h, workspace_d, workspace_bytes, q_nope_d, q_nope_stride_n,
                       q_nope_stride_h, q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d,
                       kv_scale, kv_indices_d, nullptr, &app, nullptr, nullptr, sm_scale, out_d,
                       lse_d, stream);
}

int32_t mla_merge_states(const void* v_a_d, const float* s_a_d, const void* v_b_d,
                         const float* s_b_d, void* v_out_d, float* s_out_d, int64_t num_rows,
                         int32_t head_dim, int32_t v_dtype, void* stream) {
    if (num_rows < 0 || head_dim <= 0 || head_dim % 8 != 0) return MLA_ERR_INVALID_ARG;
    if (head_dim > 4096) return MLA_ERR_UNSUPPORTED;
    if (v_dtype != MLA_DTYPE_BF16 && v_dtype != MLA_DTYPE_FP32) return MLA_ERR_UNSUPPORTED;
    if (num_rows == 0) return MLA_OK;
    if (!v_a_d || !s_a_d || !v_b_d || !s_b_d || !v_out_d || !s_out_d) return MLA_ERR_INVALID_ARG;
    if (!aligned16(v_a_d) || !aligned16(v_b_d) || !aligned16(v_out_d)) return MLA_ERR_INVALID_ARG;
    if (num_rows > (int64_t)INT32_MAX * 4) return MLA_ERR_UNSUPPORTED;
    return launch_merge_states(v_a_d, s_a_d, v_b_d, s_b_d, v_out_d, s_out_d, num_rows, head_dim,
                               v_dtype, stream) == 0
               ? MLA_OK
               : MLA_ERR_HIP;
}

namespace {

bool strides_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && a % 8 == 0 && b % 8 == 0; }

// Shared checks of the two projections: bf16 operands, head_dim 128, every
// 16-byte operand run aligned.
int32_t check_projection(const void* x, int64_t xn, int64_t xh, const void* w, int64_t w0,
                         int64_t w1, const void* y, int64_t yn, int64_t yh, int32_t num_rows,
                         int32_t num_heads, int32_t head_dim) {
    if (num_rows < 0 || num_heads <= 0 || head_dim <= 0) return MLA_ERR_INVALID_ARG;
    if (head_dim != 128 || num_heads > 65535 || num_rows > 32 * 65535) return MLA_ERR_UNSUPPORTED;
    if (num_rows == 0) return MLA_OK;
    if (!x || !w || !y || !aligned16(x) || !aligned16(w) || !aligned16(y)) return MLA_ERR_INVALID_ARG;
    if (!strides_ok(xn, xh) || !strides_ok(w0, w1) || !strides_ok(yn, yh)) return MLA_ERR_INVALID_ARG;
    return MLA_OK;
}

}  // namespace

int32_t mla_absorb_query(const void* q_d, int64_t q_stride_n, int64_t q_stride_h, const void* w_uk_d,
                         int64_t w_uk_stride_a, int64_t w_uk_stride_h, void* q_abs_d,
                         int64_t q_abs_stride_n, int64_t q_abs_stride_h, int32_t num_rows,
                         int32_t num_heads, int32_t head_dim, void* stream) {
    const int32_t err = check_projection(q_d, q_stride_n, q_stride_h, w_uk_d, w_uk_stride_a,
                                         w_uk_stride_h, q_abs_d, q_abs_stride_n, q_abs_stride_h,
                                         num_rows, num_heads, head_dim);
    if (err != MLA_OK || num_rows == 0) return err;
    HeadGemmArgs g;
    g.a = static_cast<const uint16_t*>(w_uk_d);
    g.a_head = w_uk_stride_h;
    g.a_row = w_uk_stride_a;
    g.b = static_cast<const uint16_t*>(q_d);
    g.b_head = q_stride_h;
    g.b_row = q_stride_n;
    g.d = q_abs_d;
    g.d_head = q_abs_stride_h;
    g.d_row = q_abs_stride_n;
    g.n_rows = num_rows;
    return launch_head_gemm(g, num_heads, 512, head_dim, stream) == 0 ? MLA_OK : MLA_ERR_HIP;
}

int32_t mla_project_output(const void* x_d, int64_t x_stride_n, int64_t x_stride_h, const void* w_uv_d,
                           int64_t w_uv_stride_h, int64_t w_uv_stride_d, void* o_d,
                           int64_t o_stride_n, int64_t o_stride_h, int32_t num_rows,
                           int32_t num_heads, int32_t head_dim, void* stream) {
    const int32_t err = check_projection(x_d, x_stride_n, x_stride_h, w_uv_d, w_uv_stride_h,
                                         w_uv_stride_d, o_d, o_stride_n, o_stride_h, num_rows,
                                         num_heads, head_dim);
    if (err != MLA_OK || num_rows == 0) return err;
    HeadGemmArgs g;
    g.a = static_cast<const uint16_t*>(w_uv_d);
    g.a_head = w_uv_stride_h;
    g.a_row = w_uv_stride_d;
    g.b = static_cast<const uint16_t*>(x_d);
    g.b_head = x_stride_h;
    g.b_row = x_stride_n;
    g.d = o_d;
    g.d_head = o_stride_h;
    g.d_row = o_stride_n;
    g.n_rows = num_rows;
    return launch_head_gemm(g, num_heads, head_dim, 512, stream) == 0 ? MLA_OK : MLA_ERR_HIP;
}

int32_t mla_tree_suffix_compact(const uint8_t* tree_mask_d, int64_t mask_stride,
                                const int32_t* req_to_token_d, int64_t req_stride,
                                const int32_t* prefix_lens_d, int32_t width, int32_t num_rows,
                                int32_t num_actual_rows, int32_t* page_table_d,
                                int64_t table_stride, int32_t* cache_seqlens_d, void* stream) {
    if (width < 1 || num_rows < 0 || num_actual_rows < 0 || num_actual_rows > num_rows)
        return MLA_ERR_INVALID_ARG;
    if (width > 1024) return MLA_ERR_UNSUPPORTED;
    if (num_rows == 0) return MLA_OK;
    if (!page_table_d || !cache_seqlens_d || table_stride < width) return MLA_ERR_INVALID_ARG;
    if (num_actual_rows > 0 &&
        (!tree_mask_d || !req_to_token_d || !prefix_lens_d || mask_stride < width || req_stride < width))
        return MLA_ERR_INVALID_ARG;
    return launch_tree_compact(tree_mask_d, mask_stride, req_to_token_d, req_stride, prefix_lens_d,
                               width, num_rows, num_actual_rows, page_table_d, table_stride,
                               cache_seqlens_d, stream) == 0
               ? MLA_OK
               : MLA_ERR_HIP;
}

}  // extern "C"
