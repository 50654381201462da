// Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
// planner (plan_bounds / plan_build, every params variant the library takes),
// the host index checks, and the C oracle on a small batch. Built with g++
// and the sanitizers by tests/test_sanitize_host.py; no GPU, no HIP runtime.
//
// Input: files written by the test, one batch each:
//   int32 batch, page_size, num_heads, has_qo, pool_pages, suffix_tokens,
//   then qo_indptr[batch+1] (when has_qo), kv_indptr[batch+1],
//   kv_last_page_len[batch], kv_indices[kv_indptr[batch]].
// Prints one line per batch and "ok" at the end; any sanitizer report aborts.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla_decode.h"
#include "mla_internal.h"

extern "C" {
int32_t oracle_mla_decode(int32_t batch, int32_t num_heads, int32_t page_size, const int32_t* qo_indptr,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          const int32_t* kv_last_page_len, const double* q_nope, const double* q_rope,
                          const void* cache, int32_t cache_dtype, double kv_scale, double sm_scale,
                          double* out, double* lse);
void oracle_merge_states(int64_t n, int32_t d, const double* v_a, const double* s_a, const double* v_b,
                         const double* s_b, double* v_out, double* s_out);
}

namespace {

struct Batch {
    int32_t batch = 0, page_size = 1, heads = 16, has_qo = 0, pool_pages = 0, suffix = 0;
    std::vector<int32_t> qo, kv_indptr, last, kv_indices;
};

bool read_batch(const char* path, Batch* b) {
    FILE* f = std::fopen(path, "rb");
    if (!f) return false;
    int32_t h[6];
    bool ok = std::fread(h, sizeof(int32_t), 6, f) == 6;
    b->batch = h[0], b->page_size = h[1], b->heads = h[2], b->has_qo = h[3], b->pool_pages = h[4];
    b->suffix = h[5];
    auto rd = [&](std::vector<int32_t>& v, size_t n) {
        v.resize(n);
        if (n) ok = ok && std::fread(v.data(), sizeof(int32_t), n, f) == n;
    };
    if (ok && b->has_qo) rd(b->qo, b->batch + 1);
    if (ok) rd(b->kv_indptr, b->batch + 1);
    if (ok) rd(b->last, b->batch);
    if (ok) rd(b->kv_indices, b->kv_indptr[b->batch]);
    std::fclose(f);
    return ok;
}

int plan_one(const Batch& b, mla_decode_params p, int32_t cus) {
    const int32_t rows = b.has_qo ? b.qo[b.batch] : b.batch;
    if (p.flags & MLA_DECODE_GRAPH_SAFE) p.max_rows = rows + 5;
    size_t plan_bytes = 0, ws_bytes = 0;
    int32_t st = mla::plan_bounds(&p, cus, b.batch, rows, &plan_bytes, &ws_bytes);
    if (st != MLA_OK) return st;
    std::vector<unsigned char> plan(plan_bytes);
    st = mla::plan_build(&p, cus, b.batch, b.has_qo ? b.qo.data() : nullptr, b.kv_indptr.data(),
                         b.last.data(), plan.data(), plan.size());
    if (st != MLA_OK) return st;
    const mla_plan_header* h = reinterpret_cast<const mla_plan_header*>(plan.data());
    if ((size_t)h->plan_bytes > plan_bytes || (size_t)h->workspace_bytes > ws_bytes) return 100;
    // Read every item, merge and worker entry back (ASan checks the bounds).
    const mla_work_item* items = reinterpret_cast<const mla_work_item*>(plan.data() + h->items_offset);
    const int32_t* workers = reinterpret_cast<const int32_t*>(plan.data() + h->workers_offset);
    int64_t tokens = 0;
    for (int32_t i = 0; i < h->num_items; ++i) tokens += items[i].kv_end - items[i].kv_begin;
    if (workers[h->num_workers] != h->num_items) return 101;
    const mla_merge_item* merges = reinterpret_cast<const mla_merge_item*>(plan.data() + h->merges_offset);
    for (int32_t m = 0; m < h->num_merges; ++m)
        if (merges[m].partial_begin + merges[m].num_partials > h->num_partials) return 102;
    std::printf("    H=%d ps=%d flags=%d splits=%d out=%d cus=%d: items=%d merges=%d tokens=%lld\n",
                p.num_heads, p.page_size, p.flags, p.max_splits, p.out_dtype, cus, h->num_items,
                h->num_merges, (long long)tokens);
    return MLA_OK;
}

int run_batch(const Batch& b) {
    int bad = 0;
    for (int32_t cus : {256, 13, 1}) {
        for (int variant = 0; variant < 8; ++variant) {
            mla_decode_params p{};
            p.num_heads = b.heads;
            p.kv_lora_rank = 512;
            p.qk_rope_head_dim = 64;
            p.page_size = b.page_size;
            p.kv_dtype = MLA_DTYPE_BF16;
            p.out_dtype = MLA_DTYPE_BF16;
            p.num_cus = cus;
            p.suffix_tokens = b.suffix;
            if (variant == 1) p.flags = MLA_DECODE_GRAPH_SAFE;
            if (variant == 2) p.max_splits = 1;
            if (variant == 3) p.out_dtype = MLA_DTYPE_FP32;
            if (variant == 4) {
                if (b.heads != 128 || b.suffix) continue;
                p.kv_dtype = MLA_DTYPE_FP8_E4M3FN;
                p.flags = MLA_DECODE_FP8_SCORE;
            }
            if (variant == 5) {
                if (b.heads != 128 || b.suffix) continue;
                p.kv_dtype = MLA_DTYPE_FP8_E4M3FN;
                p.flags = MLA_DECODE_FP8_SCORE | MLA_DECODE_GRAPH_SAFE;
            }
            if (variant == 6) {
                if (b.suffix) continue;
                p.flags = MLA_DECODE_SHARED_ROWS;
            }
            if (variant == 7) {
                if (b.suffix) continue;
                p.flags = MLA_DECODE_SHARED_ROWS | MLA_DECODE_GRAPH_SAFE;
            }
            const int st = plan_one(b, p, cus);
            if (st != MLA_OK) {
                std::printf("    plan failed: status %d (variant %d, cus %d)\n", st, variant, cus);
                ++bad;
            }
        }
    }
    int64_t where = -1;
    const int32_t vst = mla_decode_validate_batch(b.page_size, b.batch, b.has_qo ? b.qo.data() : nullptr,
                                                  b.kv_indptr.data(), b.kv_indices.data(), b.last.data(),
                                                  b.pool_pages, &where);
    if (vst != MLA_OK) {
        std::printf("    validate failed: %d at %lld\n", vst, (long long)where);
        ++bad;
    }
    return bad;
}

// The oracle on a small ragged batch with a few query rows per request.
int run_oracle() {
    const int32_t B = 3, H = 4, ps = 5;
    const int32_t lens[B] = {0, 7, 23};
    std::vector<int32_t> qo = {0, 1, 3, 6}, kv_indptr = {0}, last(B), kv_indices;
    int32_t next = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t np = (lens[b] + ps - 1) / ps;
        for (int32_t k = 0; k < np; ++k) kv_indices.push_back(next++);
        kv_indptr.push_back(kv_indptr.back() + np);
        last[b] = np ? lens[b] - (np - 1) * ps : 0;
    }
    const int32_t N = qo[B];
    std::vector<uint16_t> cache((size_t)next * ps * 576);
    for (size_t i = 0; i < cache.size(); ++i) cache[i] = (uint16_t)(0x3C00 + (i * 37) % 256);  // small bf16
    std::vector<double> qn((size_t)N * H * 512), qr((size_t)N * H * 64), out((size_t)N * H * 512), lse((size_t)N * H);
    for (size_t i = 0; i < qn.size(); ++i) qn[i] = std::sin(0.1 * (double)i);
    for (size_t i = 0; i < qr.size(); ++i) qr[i] = std::cos(0.3 * (double)i);
    if (oracle_mla_decode(B, H, ps, qo.data(), kv_indptr.data(), kv_indices.data(), last.data(), qn.data(),
                          qr.data(), cache.data(), 0, 1.0, 0.07, out.data(), lse.data()) != 0)
        return 1;
    std::vector<double> v(out.size()), s(lse.size());
    oracle_merge_states((int64_t)N * H, 512, out.data(), lse.data(), out.data(), lse.data(), v.data(), s.data());
    for (size_t i = 0; i < lse.size(); ++i)
        if (!(std::isinf(lse[i]) && lse[i] < 0) && !(std::fabs(s[i] - lse[i] - std::log(2.0)) < 1e-12)) return 2;
    std::printf("  oracle: %d rows, merge of a state with itself adds ln 2\n", N);
    return 0;
}

}  // namespace

int main(int argc, char** argv) {
    int bad = 0;
    for (int i = 1; i < argc; ++i) {
        Batch b;
        if (!read_batch(argv[i], &b)) {
            std::printf("cannot read %s\n", argv[i]);
            return 1;
        }
        std::printf("  %s: batch=%d H=%d ps=%d suffix=%d\n", argv[i], b.batch, b.heads, b.page_size, b.suffix);
        bad += run_batch(b);
    }
    bad += run_oracle();
    if (bad) {
        std::printf("FAILED %d\n", bad);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
