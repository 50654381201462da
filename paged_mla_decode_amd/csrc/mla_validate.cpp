// Host-side checks of a batch's index arrays against the pool (C ABI, see
// include/mla_decode.h). They read host copies only and enqueue nothing: the
// decode entry points take no pool size, so a caller that cannot vouch for its
// page numbers runs these before the call.
#include <cstdint>

#include "mla_decode.h"

namespace {

// CSR offsets: start at 0 and never decrease.
bool valid_indptr(const int32_t* indptr, int32_t n) {
    if (indptr[0] != 0) return false;
    for (int32_t i = 0; i < n; ++i)
        if (indptr[i + 1] < indptr[i]) return false;
    return true;
}

void set_bad(int64_t* bad, int64_t v) {
    if (bad) *bad = v;
}

}  // namespace

extern "C" {

int32_t mla_decode_validate_batch(int32_t page_size, int32_t batch, const int32_t* qo_indptr_h,
                                  const int32_t* kv_indptr_h, const int32_t* kv_indices_h,
                                  const int32_t* kv_last_page_len_h, int64_t num_pool_pages,
                                  int64_t* bad_entry) {
    set_bad(bad_entry, -1);
    if (page_size < 1 || batch < 0 || num_pool_pages < 0 || !kv_indptr_h) return MLA_ERR_INVALID_ARG;
    if (!valid_indptr(kv_indptr_h, batch)) return MLA_ERR_INVALID_ARG;
    if (qo_indptr_h && !valid_indptr(qo_indptr_h, batch)) return MLA_ERR_INVALID_ARG;
    const int64_t entries = kv_indptr_h[batch];
    if (entries > 0 && !kv_indices_h) return MLA_ERR_INVALID_ARG;
    for (int64_t e = 0; e < entries; ++e) {
        const int32_t page = kv_indices_h[e];
        if (page < 0 || page >= num_pool_pages) {
            set_bad(bad_entry, e);
            return MLA_ERR_INVALID_ARG;
        }
    }
    if (kv_last_page_len_h) {
        for (int32_t b = 0; b < batch; ++b) {
            if (kv_indptr_h[b + 1] == kv_indptr_h[b]) continue;  // no pages: length 0
            const int32_t last = kv_last_page_len_h[b];
            if (last < 1 || last > page_size) return MLA_ERR_INVALID_ARG;
        }
    }
    return MLA_OK;
}

int32_t mla_tree_validate_inputs(const int32_t* req_to_token_h, int64_t req_stride,
                                 int32_t num_requests, const int32_t* prefix_lens_h, int32_t width,
                                 int64_t num_pool_rows, int64_t* bad_entry) {
    set_bad(bad_entry, -1);
    if (!req_to_token_h || !prefix_lens_h || num_requests < 0 || width < 1 || req_stride < width ||
        num_pool_rows < 0)
        return MLA_ERR_INVALID_ARG;
    for (int32_t r = 0; r < num_requests; ++r) {
        const int64_t p = prefix_lens_h[r];
        if (p < 0 || p + width > req_stride) return MLA_ERR_INVALID_ARG;
        for (int32_t c = 0; c < width; ++c) {
            const int64_t at = (int64_t)r * req_stride + p + c;
            const int32_t slot = req_to_token_h[at];
            if (slot < 0 || slot >= num_pool_rows) {
                set_bad(bad_entry, at);
                return MLA_ERR_INVALID_ARG;
            }
        }
    }
    return MLA_OK;
}

int32_t mla_tree_validate_suffix(const int32_t* suffix_table_h, int64_t suffix_stride,
                                 const int32_t* suffix_lens_h, int32_t num_rows,
                                 int32_t suffix_tokens, int64_t num_pool_rows, int64_t* bad_entry) {
    set_bad(bad_entry, -1);
    if (!suffix_table_h || !suffix_lens_h || num_rows < 0 || suffix_tokens < 1 ||
        suffix_stride < suffix_tokens || num_pool_rows < 0)
        return MLA_ERR_INVALID_ARG;
    for (int32_t n = 0; n < num_rows; ++n) {
        const int32_t len = suffix_lens_h[n];
        if (len < 0) return MLA_ERR_INVALID_ARG;
        const int32_t used = len < suffix_tokens ? len : suffix_tokens;
        for (int32_t j = 0; j < used; ++j) {
            const int64_t at = (int64_t)n * suffix_stride + j;
            const int32_t slot = suffix_table_h[at];
            if (slot < 0 || slot >= num_pool_rows) {
                set_bad(bad_entry, at);
                return MLA_ERR_INVALID_ARG;
            }
        }
    }
    return MLA_OK;
}

}  // extern "C"
