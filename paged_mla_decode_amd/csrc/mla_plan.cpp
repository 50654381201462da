// Host planner for absorbed-MLA paged decode: split-KV chunking and balance
// across compute units.
//
// The batch arrives as CSR page lists (the "Paged, ragged batches" paragraph of
// the SGLang attention-backends page). Like the plan() that page describes, this
// runs on the host once per batch, picks how many chunks each query row's KV is
// split into, and balances long and short requests across the chip; the
// result is reused by every layer. Pure host code: no HIP calls.
//
// Policy:
//   * Total work T = sum over query rows of their token counts. With G
//     workgroups resident at once (compute units x workgroups per CU), the
//     target chunk is ceil(T / G) tokens, never below the variant's min_chunk
//     (a partial costs H*512 values, bf16 or fp32, written and read back, plus a second load
//     of the query), rounded up to the 32-token tile.
//   * A row longer than the target is cut into equal tile-aligned chunks
//     (at most max_splits). Short rows stay whole and write their output
//     directly; only split rows use partial slots and a merge.
//   * Work items are ordered longest first, so the hardware dispatcher, which
//     hands workgroups to CUs as they free up, approximates longest-processing-
//     time-first scheduling.
#include <algorithm>
#include <cstring>
#include <vector>

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kDefaultMaxSplits = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool select_variant(const mla_decode_params* p, Variant* v) {
    if (!p) return false;
    if (p->kv_lora_rank != kLatent || p->qk_rope_head_dim != kRope || p->page_size < 1) return false;
    if (p->kv_dtype != MLA_DTYPE_BF16 && p->kv_dtype != MLA_DTYPE_FP8_E4M3FN) return false;
    if (p->out_dtype != MLA_DTYPE_BF16 && p->out_dtype != MLA_DTYPE_FP32) return false;
    switch (p->num_heads) {
        case 128: *v = Variant{32, 4, 1, 512}; return true;
        case 64: *v = Variant{16, 4, 1, 256}; return true;
        case 32: *v = Variant{16, 2, 1, 128}; return true;
        case 16: *v = Variant{16, 1, 2, 128}; return true;
        default: return false;
    }
}

const char* variant_name(const mla_decode_params* p) {
    Variant v;
    if (!select_variant(p, &v)) return nullptr;
    const bool kv8 = p->kv_dtype == MLA_DTYPE_FP8_E4M3FN;
    const bool o32 = p->out_dtype == MLA_DTYPE_FP32;
    static const char* names[2][3][2][2] = {
        {{{"mla_decode<hw16,hs1,kv_bf16,out_bf16>", "mla_decode<hw16,hs1,kv_bf16,out_fp32>"},
          {"mla_decode<hw16,hs1,kv_fp8,out_bf16>", "mla_decode<hw16,hs1,kv_fp8,out_fp32>"}},
         {{"mla_decode<hw16,hs2,kv_bf16,out_bf16>", "mla_decode<hw16,hs2,kv_bf16,out_fp32>"},
          {"mla_decode<hw16,hs2,kv_fp8,out_bf16>", "mla_decode<hw16,hs2,kv_fp8,out_fp32>"}},
         {{"mla_decode<hw16,hs4,kv_bf16,out_bf16>", "mla_decode<hw16,hs4,kv_bf16,out_fp32>"},
          {"mla_decode<hw16,hs4,kv_fp8,out_bf16>", "mla_decode<hw16,hs4,kv_fp8,out_fp32>"}}},
        {{{nullptr, nullptr}, {nullptr, nullptr}},
         {{nullptr, nullptr}, {nullptr, nullptr}},
         {{"mla_decode<hw32,hs4,kv_bf16,out_bf16>", "mla_decode<hw32,hs4,kv_bf16,out_fp32>"},
          {"mla_decode<hw32,hs4,kv_fp8,out_bf16>", "mla_decode<hw32,hs4,kv_fp8,out_fp32>"}}}};
    const int hsi = v.hs == 1 ? 0 : (v.hs == 2 ? 1 : 2);
    return names[v.hw == 32 ? 1 : 0][hsi][kv8][o32];
}

// Partials are stored in the output's precision: bf16, or fp32 in the fp32 mode.
static int64_t partial_elem_bytes(const mla_decode_params* p) { return p->out_dtype == MLA_DTYPE_FP32 ? 4 : 2; }

static void layout(int32_t num_items, int32_t num_merges, int32_t num_partials, int32_t num_heads,
                   int64_t elem_bytes, mla_plan_header* h) {
    h->items_offset = align_up(sizeof(mla_plan_header), 64);
    h->merges_offset = align_up(h->items_offset + (int64_t)num_items * sizeof(mla_work_item), 64);
    h->plan_bytes = align_up(h->merges_offset + (int64_t)num_merges * sizeof(mla_merge_item), 256);
    h->partial_out_offset = h->plan_bytes;
    h->partial_lse_offset =
        align_up(h->partial_out_offset + (int64_t)num_partials * num_heads * kLatent * elem_bytes, 256);
    h->workspace_bytes = align_up(h->partial_lse_offset + (int64_t)num_partials * num_heads * 4, 256);
}

int32_t plan_bounds(const mla_decode_params* p, int32_t num_cus, int32_t batch, int32_t num_rows,
                    size_t* plan_bytes, size_t* workspace_bytes) {
    Variant v;
    if (!p || batch < 0 || num_rows < 0 || num_cus <= 0) return MLA_ERR_INVALID_ARG;
    if (!select_variant(p, &v)) return MLA_ERR_UNSUPPORTED;
    // Chunks: at most one per row plus ceil(T / chunk) <= G extra; split rows
    // hold at most 2 * T / chunk <= 2G partials.
    const int64_t G = (int64_t)num_cus * v.wgs_per_cu;
    const int64_t items = (int64_t)num_rows + G + 1;
    const int64_t partials = std::min<int64_t>(items, 2 * G + 2);
    mla_plan_header h{};
    layout((int32_t)items, num_rows, (int32_t)partials, p->num_heads, partial_elem_bytes(p), &h);
    if (plan_bytes) *plan_bytes = (size_t)h.plan_bytes;
    if (workspace_bytes) *workspace_bytes = (size_t)h.workspace_bytes;
    return MLA_OK;
}

int32_t plan_build(const mla_decode_params* p, int32_t num_cus, int32_t batch,
                   const int32_t* qo_indptr, const int32_t* kv_indptr,
                   const int32_t* kv_last_page_len, void* plan_h, size_t plan_h_bytes) {
    Variant v;
    if (!p || batch < 0 || num_cus <= 0 || !kv_indptr || !plan_h) return MLA_ERR_INVALID_ARG;
    if (!select_variant(p, &v)) return MLA_ERR_UNSUPPORTED;
    const int ps = p->page_size;

    // Validate the CSR arrays and compute each request's length.
    if (kv_indptr[0] < 0) return MLA_ERR_INVALID_ARG;
    if (qo_indptr && qo_indptr[0] != 0) return MLA_ERR_INVALID_ARG;
    std::vector<int64_t> len(batch);
    int64_t num_rows = 0, total = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t np = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        if (np < 0) return MLA_ERR_INVALID_ARG;
        int64_t L = 0;
        if (np > 0) {
            const int64_t last = kv_last_page_len ? kv_last_page_len[b] : ps;
            if (last < 1 || last > ps) return MLA_ERR_INVALID_ARG;
            L = (np - 1) * ps + last;
        }
        if (L > INT32_MAX - kTile) return MLA_ERR_UNSUPPORTED;
        len[b] = L;
        const int64_t rows = qo_indptr ? (int64_t)qo_indptr[b + 1] - qo_indptr[b] : 1;
        if (rows < 0) return MLA_ERR_INVALID_ARG;
        num_rows += rows;
        total += rows * L;
    }
    if (num_rows > INT32_MAX) return MLA_ERR_UNSUPPORTED;

    const int64_t G = (int64_t)num_cus * v.wgs_per_cu;
    int64_t chunk = std::max<int64_t>(v.min_chunk, (total + G - 1) / std::max<int64_t>(G, 1));
    chunk = align_up(chunk, kTile);
    const int64_t max_splits = p->max_splits > 0 ? p->max_splits : kDefaultMaxSplits;

    std::vector<mla_work_item> items;
    std::vector<mla_merge_item> merges;
    items.reserve((size_t)(num_rows + G + 1));
    int32_t num_partials = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t r0 = qo_indptr ? qo_indptr[b] : b;
        const int64_t r1 = qo_indptr ? qo_indptr[b + 1] : b + 1;
        const int64_t L = len[b];
        int64_t n = std::max<int64_t>(1, std::min<int64_t>(max_splits, (L + chunk - 1) / chunk));
        const int64_t step = n > 1 ? align_up((L + n - 1) / n, kTile) : L;
        if (n > 1) n = (L + step - 1) / step;  // tile alignment can drop a chunk
        for (int64_t r = r0; r < r1; ++r) {
            const int32_t first_partial = n > 1 ? num_partials : -1;
            for (int64_t c = 0; c < n; ++c) {
                mla_work_item it{};
                it.row = (int32_t)r;
                it.request = b;
                it.page_base = kv_indptr[b];
                it.kv_begin = (int32_t)(c * step);
                it.kv_end = (int32_t)std::min<int64_t>(L, (c + 1) * step);
                it.partial = n > 1 ? num_partials++ : -1;
                it.head_begin = 0;
                it.num_heads = p->num_heads;
                items.push_back(it);
            }
            if (n > 1) merges.push_back(mla_merge_item{(int32_t)r, first_partial, (int32_t)n, 0});
        }
    }
    // Longest chunks first (stable, so equal chunks keep row order).
    std::stable_sort(items.begin(), items.end(), [](const mla_work_item& x, const mla_work_item& y) {
        return (x.kv_end - x.kv_begin) > (y.kv_end - y.kv_begin);
    });

    mla_plan_header h{};
    h.magic = MLA_PLAN_MAGIC;
    h.version = MLA_PLAN_VERSION;
    h.num_heads = p->num_heads;
    h.page_size = ps;
    h.kv_dtype = p->kv_dtype;
    h.out_dtype = p->out_dtype;
    h.batch = batch;
    h.num_rows = (int32_t)num_rows;
    h.num_items = (int32_t)items.size();
    h.num_merges = (int32_t)merges.size();
    h.num_partials = num_partials;
    h.chunk_tokens = (int32_t)chunk;
    h.num_page_entries = kv_indptr[batch];
    layout(h.num_items, h.num_merges, num_partials, p->num_heads, partial_elem_bytes(p), &h);
    if ((size_t)h.plan_bytes > plan_h_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;

    char* dst = static_cast<char*>(plan_h);
    std::memset(dst, 0, (size_t)h.plan_bytes);
    std::memcpy(dst, &h, sizeof h);
    if (!items.empty())
        std::memcpy(dst + h.items_offset, items.data(), items.size() * sizeof(mla_work_item));
    if (!merges.empty())
        std::memcpy(dst + h.merges_offset, merges.data(), merges.size() * sizeof(mla_merge_item));
    return MLA_OK;
}

}  // namespace mla
