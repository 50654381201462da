// Host planner for absorbed-MLA paged decode: split-KV chunking and balance
// across compute units.
//
// The batch arrives as CSR page lists (the "Paged, ragged batches" paragraph of
// the SGLang attention-backends page). Like the plan() that page describes, this
// runs on the host once per batch, picks how many chunks each query row's KV is
// split into, and balances long and short requests across the chip; the
// result is reused by every layer. Pure host code: no HIP calls.
//
// Policy: persistent workers with an equal-work fill.
//   * The decode launch has one workgroup per worker: G = compute units x
//     workgroups per CU, all resident at once. Each worker processes the list
//     of work items the plan gives it, in order.
//   * Work is measured in 32-token tiles. A work item (one query row, one
//     contiguous token range) costs its tiles plus the kernel's item cost, the fixed cost of
//     starting and finishing an item (query load, first-tile latency, output
//     store).
//   * Rows are taken longest first and poured into workers up to a capacity C:
//     a row that does not fit is cut at the worker boundary and continues on
//     the next worker. C is the smallest capacity (binary search) for which
//     the fill needs at most G workers, so every worker gets about the same
//     work and a row is split only where a worker boundary falls into it.
//   * No piece is shorter than the item cost unless its row is (a worker may
//     exceed C by that much rather than cut one off); a row is cut into at
//     most max_splits pieces. A split row's pieces write
//     partials (in the output precision) that one merge combines.
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
    if (!p || (p->flags & ~(MLA_DECODE_GRAPH_SAFE | MLA_DECODE_FP8_SCORE | MLA_DECODE_SHARED_ROWS)) != 0)
        return false;
    // The fp8 score: the 128-head kernel over an e4m3fn cache, bf16 output, plain decode.
    if ((p->flags & MLA_DECODE_FP8_SCORE) &&
        (p->num_heads != 128 || p->kv_dtype != MLA_DTYPE_FP8_E4M3FN || p->out_dtype != MLA_DTYPE_BF16 ||
         p->suffix_tokens != 0))
        return false;
    // Single-pass tree verify: the 128-head kernel over token slots (page size 1).
    if (p->suffix_tokens < 0 || p->suffix_tokens > kMaxSuffixTokens) return false;
    if (p->suffix_tokens > 0 && (p->num_heads != 128 || p->page_size != 1)) return false;
    if (p->kv_lora_rank != kLatent || p->qk_rope_head_dim != kRope || p->page_size < 1) return false;
    if (p->kv_dtype != MLA_DTYPE_BF16 && p->kv_dtype != MLA_DTYPE_FP8_E4M3FN) return false;
    if (p->out_dtype != MLA_DTYPE_BF16 && p->out_dtype != MLA_DTYPE_FP32) return false;
    // Shared rows: 64 / H rows of 16 or 32 heads per item, on the 64-head kernel.
    if ((p->flags & MLA_DECODE_SHARED_ROWS) && (p->num_heads == 16 || p->num_heads == 32)) {
        *v = Variant{16, 4, 1, 4, 64 / p->num_heads};
        return true;
    }
    switch (p->num_heads) {
        // The 128-head kernel loads a 144 KiB query and stores a 128 KiB output
        // per item, about as long as 8 tiles of its main loop; the smaller
        // kernels' items cost about 4.
        case 128: *v = Variant{32, 4, 1, 8}; return true;
        case 64: *v = Variant{16, 4, 1, 4}; return true;
        case 32: *v = Variant{16, 2, 1, 4}; return true;
        // 16 heads: a second, load-only wave halves each wave's loads per tile,
        // so that four stages fit the vmcnt budget (one workgroup per CU).
        case 16: *v = Variant{16, 2, 1, 4}; return true;
        default: return false;
    }
}

const char* variant_name(const mla_decode_params* p) {
    Variant v;
    if (!select_variant(p, &v)) return nullptr;
    if (p->flags & MLA_DECODE_FP8_SCORE) return "mla_decode<hw32,hs4,kv_fp8,out_bf16,score_fp8>";
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

// q_rows: rows of the quantised query (fp8 score), 0 without it.
static void layout(int32_t num_items, int32_t num_merges, int32_t num_workers, int32_t num_partials,
                   int32_t num_heads, int64_t elem_bytes, int32_t q_rows, mla_plan_header* h) {
    h->items_offset = align_up(sizeof(mla_plan_header), 64);
    h->merges_offset = align_up(h->items_offset + (int64_t)num_items * sizeof(mla_work_item), 64);
    h->workers_offset = align_up(h->merges_offset + (int64_t)num_merges * sizeof(mla_merge_item), 64);
    h->plan_bytes = align_up(h->workers_offset + ((int64_t)num_workers + 1) * 4, 256);
    h->partial_out_offset = h->plan_bytes;
    h->partial_lse_offset =
        align_up(h->partial_out_offset + (int64_t)num_partials * num_heads * kLatent * elem_bytes, 256);
    h->workspace_bytes = align_up(h->partial_lse_offset + (int64_t)num_partials * num_heads * 4, 256);
    h->query_codes_offset = h->query_exp_offset = 0;
    if (q_rows > 0) {
        h->query_codes_offset = h->workspace_bytes;
        h->query_exp_offset = align_up(h->query_codes_offset + (int64_t)q_rows * num_heads * (kLatent + kRope), 256);
        h->workspace_bytes = align_up(h->query_exp_offset + (int64_t)q_rows * num_heads * 4, 256);
    }
}
static int32_t query_rows(const mla_decode_params* p, int32_t rows) {
    return (p->flags & MLA_DECODE_FP8_SCORE) ? rows : 0;
}

int32_t plan_bounds(const mla_decode_params* p, int32_t num_cus, int32_t batch, int32_t num_rows,
                    size_t* plan_bytes, size_t* workspace_bytes) {
    Variant v;
    if (!p || batch < 0 || num_rows < 0 || num_cus <= 0) return MLA_ERR_INVALID_ARG;
    if (!select_variant(p, &v)) return MLA_ERR_UNSUPPORTED;
    // Items: one per row plus at most one extra per worker boundary (G - 1);
    // the pieces of split rows are at most 2 (G - 1).
    const int64_t G = (int64_t)num_cus * v.wgs_per_cu;
    // Graph-safe plans are laid out for params.max_rows rows.
    if (p->flags & MLA_DECODE_GRAPH_SAFE) {
        if (p->max_rows < 1) return MLA_ERR_INVALID_ARG;
        num_rows = std::max(num_rows, p->max_rows);
    }
    const int64_t items = (int64_t)num_rows + G + 1;
    // A split item writes one partial per query row it holds.
    const int64_t partials = std::min<int64_t>(items, 2 * G + 2) * v.rows_per_item;
    mla_plan_header h{};
    layout((int32_t)items, num_rows, (int32_t)G, (int32_t)partials, p->num_heads, partial_elem_bytes(p),
           query_rows(p, num_rows), &h);
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
        L += p->suffix_tokens;  // tree verify: room for each row's suffix slots
        if (L > INT32_MAX - kTile) return MLA_ERR_UNSUPPORTED;
        len[b] = L;
        const int64_t rows = qo_indptr ? (int64_t)qo_indptr[b + 1] - qo_indptr[b] : 1;
        if (rows < 0) return MLA_ERR_INVALID_ARG;
        num_rows += rows;
        total += rows * L;
    }
    if (num_rows > INT32_MAX) return MLA_ERR_UNSUPPORTED;

    const int64_t G = std::max<int64_t>(1, (int64_t)num_cus * v.wgs_per_cu);
    const int64_t max_splits = p->max_splits > 0 ? p->max_splits : kDefaultMaxSplits;
    const int64_t item_cost = v.item_cost;
    // Shortest piece: the item cost (a piece at least as long as its fixed
    // cost), or two tiles where that lowers the capacity (below).
    int64_t min_piece = item_cost;
    const int64_t sfx = p->suffix_tokens;

    // The planned units: a query row, or with shared rows up to rows_per_item
    // consecutive rows of one request (they read the same tokens).
    struct Row {
        int32_t row, request;
        int64_t len, tiles;
        int32_t nrows;
    };
    const int64_t R = v.rows_per_item;
    std::vector<Row> rows;
    rows.reserve((size_t)num_rows);
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t r0 = qo_indptr ? qo_indptr[b] : b;
        const int64_t r1 = qo_indptr ? qo_indptr[b + 1] : b + 1;
        for (int64_t r = r0; r < r1; r += R)
            rows.push_back(Row{(int32_t)r, b, len[b], (len[b] + kTile - 1) / kTile, (int32_t)std::min(R, r1 - r)});
    }
    std::stable_sort(rows.begin(), rows.end(), [](const Row& x, const Row& y) { return x.tiles > y.tiles; });

    struct Piece {
        int32_t row_index, worker;
        int64_t t0, t1;  // tile range
    };
    // Pour the rows into workers of capacity C; false if more than G are needed.
    auto fill = [&](int64_t C, std::vector<Piece>* out) {
        if (out) out->clear();
        int64_t w = 0, load = 0;
        for (size_t i = 0; i < rows.size(); ++i) {
            int64_t rem = rows[i].tiles, t = 0, pieces = 0;
            for (;;) {  // at least one piece, also for an empty row
                const bool last_allowed = pieces + 1 >= max_splits;  // this piece takes the rest
                const int64_t cap = C - load - item_cost;
                if (load > 0 && (cap < std::min(min_piece, rem) || (last_allowed && rem > cap))) {
                    if (++w >= G) return false;
                    load = 0;
                    continue;
                }
                int64_t take = last_allowed ? rem : std::min(rem, std::max<int64_t>(cap, 1));
                // Neither this piece nor the rest of the row shorter than min_piece,
                // where the row allows it.
                if (take < rem && rem - take < min_piece) take = rem >= 2 * min_piece ? rem - min_piece : rem;
                if (take < rem && take < min_piece) take = std::min(rem, min_piece);
                // Tree verify: no cut inside a row's last suffix_tokens tokens, so
                // that its last chunk holds every suffix slot.
                if (sfx > 0 && take < rem && (t + take) * kTile > rows[i].len - sfx) {
                    const int64_t cut = (rows[i].len - sfx) / kTile;
                    take = cut > t ? cut - t : rem;
                }
                if (out) out->push_back(Piece{(int32_t)i, (int32_t)w, t, t + take});
                t += take;
                rem -= take;
                load += take + item_cost;
                ++pieces;
                if (rem == 0) break;
                if (++w >= G) return false;
                load = 0;
            }
        }
        return true;
    };
    // The least capacity with which the pour fits G workers.
    auto search = [&]() {
        int64_t hi = item_cost;
        for (const Row& r : rows) hi += r.tiles + item_cost;
        int64_t lo = 0;  // infeasible (no capacity)
        while (hi - lo > 1) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (fill(mid, nullptr))
                hi = mid;
            else
                lo = mid;
        }
        return hi;
    };
    int64_t hi = search();
    // With the item cost as the shortest piece a worker moves on while up to
    // twice that much capacity is left, so the search can settle a tile or more
    // above the average load and leave workers idle (12 of 256 on a 64-row,
    // 16-head batch). Two-tile pieces fill those gaps; they are kept only where
    // they lower the capacity, since otherwise they only add items (each loads
    // the query and writes an output): measured on three workloads, a
    // 2-4% gain where the capacity fell and a 2% loss where it did not.
    if (item_cost > 2) {
        min_piece = 2;
        const int64_t hi2 = search();
        if (hi2 < hi)
            hi = hi2;
        else
            min_piece = item_cost;
    }
    std::vector<Piece> pieces;
    if (!fill(hi, &pieces)) return MLA_ERR_UNSUPPORTED;  // unreachable: hi is feasible

    // Partial slots: the pieces of a split unit take consecutive runs of slots,
    // one slot per row (piece c of a unit of n rows: slots first + c n + r), so
    // that row r's partials are first + r + k n, k < pieces.
    std::vector<int32_t> npieces(rows.size(), 0), first_slot(rows.size(), -1);
    for (const Piece& pc : pieces) ++npieces[pc.row_index];
    std::vector<mla_merge_item> merges;
    int32_t num_partials = 0;
    for (size_t i = 0; i < rows.size(); ++i)
        if (npieces[i] > 1) {
            first_slot[i] = num_partials;
            for (int32_t r = 0; r < rows[i].nrows; ++r)
                merges.push_back(mla_merge_item{rows[i].row + r, num_partials + r, npieces[i], rows[i].nrows});
            num_partials += npieces[i] * rows[i].nrows;
        }
    // Rows with the most partials first: the merge launch takes the leading ones
    // (at least kWideMergePartials each) with a workgroup per row and head.
    std::stable_sort(merges.begin(), merges.end(),
                     [](const mla_merge_item& x, const mla_merge_item& y) { return x.num_partials > y.num_partials; });
    std::vector<int32_t> next_slot(first_slot);
    // Items per worker in pour order (pieces of a row get their partial slots in
    // token order).
    std::vector<std::vector<mla_work_item>> per_worker;
    for (const Piece& pc : pieces) {
        const Row& r = rows[pc.row_index];
        if ((size_t)pc.worker >= per_worker.size()) per_worker.resize((size_t)pc.worker + 1);
        mla_work_item it{};
        it.row = r.row;
        it.request = r.request;
        it.page_base = kv_indptr[r.request];
        it.kv_begin = (int32_t)(pc.t0 * kTile);
        it.kv_end = (int32_t)std::min<int64_t>(r.len, pc.t1 * kTile);
        it.partial = -1;
        if (npieces[pc.row_index] > 1) {
            it.partial = next_slot[pc.row_index];
            next_slot[pc.row_index] += r.nrows;
        }
        it.head_begin = 0;
        it.num_rows = r.nrows;
        it.flags = (r.len > 0 && it.kv_end == r.len) ? MLA_ITEM_LAST_CHUNK : 0u;
        per_worker[(size_t)pc.worker].push_back(it);
    }
    // Worker order. The device hands workgroups to its XCDs round robin
    // (workgroup p to XCD p % 8), each XCD with its own L2. The pour fills
    // workers with consecutive rows, and the rows of one request (several query
    // rows, a long row's pieces) are consecutive, so consecutive pour workers go
    // to one XCD: pour worker v runs as workgroup p with
    // v = (p % 8) * (G / 8) + p / 8. Tiles that several of them read then meet
    // in one L2. The launch then has all G workers, as graph-safe plans do
    // anyway; those without work exit at once.
    const int64_t used = (int64_t)per_worker.size();
    const bool by_xcd = G % kXcds == 0;
    const int64_t nw = (by_xcd || (p->flags & MLA_DECODE_GRAPH_SAFE)) ? G : used;
    std::vector<mla_work_item> items;
    items.reserve(pieces.size());
    std::vector<int32_t> worker_begin;
    for (int64_t w = 0; w < nw; ++w) {
        const int64_t v = by_xcd ? (w % kXcds) * (G / kXcds) + w / kXcds : w;
        worker_begin.push_back((int32_t)items.size());
        if (v < used) items.insert(items.end(), per_worker[(size_t)v].begin(), per_worker[(size_t)v].end());
    }
    const int32_t num_workers = (int32_t)nw;
    worker_begin.push_back((int32_t)items.size());
    const int64_t chunk = hi * kTile;

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
    h.chunk_tokens = (int32_t)std::min<int64_t>(chunk, INT32_MAX);
    h.num_workers = num_workers;
    h.max_merge_partials = 0;
    for (const mla_merge_item& mi : merges) {
        h.max_merge_partials = std::max(h.max_merge_partials, mi.num_partials);
        if (mi.num_partials >= kWideMergePartials) ++h.num_wide_merges;
    }
    h.flags = p->flags;
    h.suffix_tokens = p->suffix_tokens;
    // Tiles are read once per launch when no request has more rows than one
    // planned unit holds (pieces of one unit read disjoint tokens).
    h.tiles_read_once = 1;
    for (int32_t b = 0; qo_indptr && b < batch; ++b)
        if ((int64_t)qo_indptr[b + 1] - qo_indptr[b] > R) h.tiles_read_once = 0;
    h.num_page_entries = kv_indptr[batch];
    if (p->flags & MLA_DECODE_GRAPH_SAFE) {
        // The layout of plan_bounds for max_rows rows: the same offsets for every
        // plan of these params, so that captured launches find each array.
        if (p->max_rows < 1 || num_rows > p->max_rows) return MLA_ERR_INVALID_ARG;
        const int64_t cap_items = (int64_t)p->max_rows + G + 1;
        layout((int32_t)cap_items, p->max_rows, (int32_t)G,
               (int32_t)(std::min<int64_t>(cap_items, 2 * G + 2) * R), p->num_heads, partial_elem_bytes(p),
               query_rows(p, p->max_rows), &h);
    } else {
        layout(h.num_items, h.num_merges, num_workers, num_partials, p->num_heads, partial_elem_bytes(p),
               query_rows(p, h.num_rows), &h);
    }
    if ((size_t)h.plan_bytes > plan_h_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;

    char* dst = static_cast<char*>(plan_h);
    std::memset(dst, 0, (size_t)h.plan_bytes);
    std::memcpy(dst, &h, sizeof h);
    if (!items.empty())
        std::memcpy(dst + h.items_offset, items.data(), items.size() * sizeof(mla_work_item));
    if (!merges.empty())
        std::memcpy(dst + h.merges_offset, merges.data(), merges.size() * sizeof(mla_merge_item));
    std::memcpy(dst + h.workers_offset, worker_begin.data(), worker_begin.size() * sizeof(int32_t));
    return MLA_OK;
}

}  // namespace mla
