"""Host planner invariants (no GPU): every (query row, token) is covered by
exactly one work item, chunks stay inside their request and start on a tile
boundary, split rows map to consistent partial slots and merges, the worker
table partitions the items, and the workers' loads are balanced. Several plans
are correct; the kernel's result does not depend on which one is chosen, so
the plan is pinned by these properties rather than by equality."""
import numpy as np
import pytest

import paged_mla_decode_amd as m
import workloads

TILE = 32


def build(p, batch):
    pb, _ = m.mla_decode_workspace_size(p, batch.batch, batch.num_rows)
    plan = np.zeros(pb, np.uint8)
    qo = None if np.array_equal(batch.qo_indptr, np.arange(batch.batch + 1)) else batch.qo_indptr
    st = m.mla_decode_plan(p, batch.batch, qo, batch.kv_indptr, batch.kv_last_page_len, plan, pb)
    assert st == m.MLA_OK, m.mla_status_string(st)
    return m.read_plan(plan)


def item_cost(num_heads):
    """The planner's fixed cost per work item, in tiles (per kernel)."""
    return 8 if num_heads == 128 else 4


def rows_per_item(p):
    """Query rows of one request a work item holds."""
    if p.flags & m.MLA_DECODE_SHARED_ROWS and p.num_heads in (16, 32):
        return 64 // p.num_heads
    return 1


def worker_loads(items, workers, cost):
    return [sum(-(-(it.kv_end - it.kv_begin) // TILE) + cost for it in items[workers[w]:workers[w + 1]])
            for w in range(len(workers) - 1)]


def check_invariants(p, batch, h, items, merges, workers):
    assert h.magic == m._binding.MLA_PLAN_MAGIC and h.num_items == len(items)
    assert h.num_rows == batch.num_rows and h.batch == batch.batch
    assert h.num_page_entries == batch.kv_indptr[-1]
    lens = batch.row_seq_lens
    row_req = np.repeat(np.arange(batch.batch), np.diff(batch.qo_indptr))
    covered = {}
    partial_of = {}
    R = rows_per_item(p)
    per_req = np.diff(batch.qo_indptr)
    assert h.tiles_read_once == int(per_req.max(initial=0) <= R)
    for it in items:
        # an item holds rows it.row .. it.row + num_rows - 1 of one request
        assert 1 <= it.num_rows <= R
        rows = range(it.row, it.row + it.num_rows)
        assert 0 <= it.row and it.row + it.num_rows <= batch.num_rows
        assert all(row_req[r] == it.request for r in rows)
        assert it.page_base == batch.kv_indptr[it.request]
        assert 0 <= it.kv_begin <= it.kv_end <= lens[it.row]
        assert it.kv_begin % TILE == 0
        assert it.head_begin == 0
        # The last-chunk flag marks exactly the item that ends at a non-empty row's length.
        assert bool(it.flags & m.MLA_ITEM_LAST_CHUNK) == (lens[it.row] > 0 and it.kv_end == lens[it.row])
        assert it.flags & ~m.MLA_ITEM_LAST_CHUNK == 0
        for k, r in enumerate(rows):
            covered.setdefault(r, []).append((it.kv_begin, it.kv_end))
            if it.partial >= 0:  # row it.row + k writes slot it.partial + k
                assert it.partial + k not in partial_of
                partial_of[it.partial + k] = (it, r)
    # exact cover of every row's tokens
    for r in range(batch.num_rows):
        segs = sorted(covered[r])
        assert segs[0][0] == 0 and segs[-1][1] == lens[r]
        for (a0, a1), (b0, b1) in zip(segs, segs[1:]):
            assert a1 == b0
    # split rows <=> merge items over consecutive partial slots
    assert len(partial_of) == h.num_partials
    merged_rows = set()
    for mi in merges:
        merged_rows.add(mi.row)
        assert mi.num_partials >= 2 and mi.partial_stride >= 1
        chunks = [partial_of[mi.partial_begin + k * mi.partial_stride] for k in range(mi.num_partials)]
        assert all(r == mi.row for _, r in chunks)
        assert [(c.kv_begin, c.kv_end) for c, _ in chunks] == sorted(covered[mi.row]), "token order"
    for r, segs in covered.items():
        assert (len(segs) > 1) == (r in merged_rows)
    assert h.num_merges == len(merges)
    assert h.max_merge_partials == max((mi.num_partials for mi in merges), default=0)
    assert all(a.num_partials >= b.num_partials for a, b in zip(merges, merges[1:])), "most partials first"
    # the worker table partitions the items, at most one worker per resident workgroup
    assert len(workers) == h.num_workers + 1 and workers[0] == 0 and workers[-1] == len(items)
    assert all(a <= b for a, b in zip(workers, workers[1:]))
    G = max(1, p.num_cus)  # one workgroup per CU for every head count
    busy = [w for w in range(h.num_workers) if workers[w + 1] > workers[w]]
    if G % 8 == 0:
        # XCD order: pour worker v runs as workgroup w with v = (w % 8) * (G / 8) + w / 8,
        # so the busy workgroups are the first pour workers, a request's rows on one XCD.
        assert h.num_workers == G
        pour = sorted((w % 8) * (G // 8) + w // 8 for w in busy)
        assert pour == list(range(len(busy))), "busy workers are a prefix of the pour"
    elif p.flags & m.MLA_DECODE_GRAPH_SAFE:
        # graph-safe plans list all G workers; the busy ones come first
        assert h.num_workers == G and busy == list(range(len(busy)))
    else:
        assert busy == list(range(h.num_workers)), "every worker has an item"
    if p.flags & m.MLA_DECODE_GRAPH_SAFE:
        # The fixed merge grid of a graph-safe launch covers any plan: at most G - 1
        # split units (each crosses a worker boundary), at most ceil((G - 1) / 15)
        # of them wide, each of up to rows_per_item rows.
        R = rows_per_item(p)
        assert h.num_merges <= max(1, G - 1) * R
        assert h.num_wide_merges <= max(1, (G - 1 + 14) // 15) * R
    assert h.num_workers <= G
    # no worker above the plan's capacity by more than a minimum piece, unless
    # a single item (or an unsplittable row) forces it
    cap = h.chunk_tokens // TILE
    cost = item_cost(p.num_heads)
    for w, load in enumerate(worker_loads(items, workers, cost)):
        n = workers[w + 1] - workers[w]
        if load > cap + cost:
            assert n == 1 or p.max_splits > 0, (w, load, cap)


@pytest.mark.parametrize("make,H,ps", [
    (lambda: workloads.v3(), 128, 64),
    (lambda: workloads.v2_lite(), 16, 1),
    (lambda: workloads.random_decode_batch(1, [0, 1, 31, 32, 33, 5000, 0, 70000], 128, 16), 128, 16),
    (lambda: workloads.random_decode_batch(2, [7, 33], 16, 1, rows_per_request=3), 16, 1),
])
def test_plan_invariants(make, H, ps):
    batch = make()
    for cus, splits in ((256, 0), (256, 1), (80, 3), (1, 0)):
        p = m.make_params(H, ps, num_cus=cus, max_splits=splits)
        h, items, merges, workers = build(p, batch)
        check_invariants(p, batch, h, items, merges, workers)
        if splits == 1:
            assert h.num_merges == 0 and h.num_partials == 0


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, [0, 4, 1, 9, 2, 0, 3]])
def test_shared_rows_plan_invariants(H, rows):
    """MLA_DECODE_SHARED_ROWS: up to 64 / H consecutive rows of a request per
    item (16 and 32 heads; one row otherwise), each row's pieces in its own
    partial slots, a merge per split row over strided slots."""
    lens = [0, 40, 300, 1, 2048, 64, 5000]
    nb = len(lens)
    batch = workloads.random_decode_batch(5, lens, H, 16, rows_per_request=rows)
    for cus, splits in ((256, 0), (64, 0), (80, 3), (1, 0)):
        p = m.make_params(H, 16, num_cus=cus, max_splits=splits, flags=m.MLA_DECODE_SHARED_ROWS)
        h, items, merges, workers = build(p, batch)
        check_invariants(p, batch, h, items, merges, workers)
        R = rows_per_item(p)
        per_req = np.diff(batch.qo_indptr)
        # every request's rows form ceil(rows / R) units, each planned like one row
        units = sum(-(-int(n) // R) for n in per_req)
        firsts = {(it.request, it.row) for it in items}
        assert len(firsts) == units, (len(firsts), units)
    assert nb == batch.batch


def test_shared_rows_graph_safe_layout_holds_every_plan():
    """Graph-safe shared-rows plans keep one layout, with room for a partial per
    row of every split unit."""
    p = m.make_params(16, 1, num_cus=256, flags=m.MLA_DECODE_SHARED_ROWS | m.MLA_DECODE_GRAPH_SAFE, max_rows=64)
    offs = set()
    for rows in (1, 4, [4, 3, 2, 1] * 4):
        batch = workloads.random_decode_batch(6, [3000] * 16, 16, 1, rows_per_request=rows)
        h, items, merges, workers = build(p, batch)
        check_invariants(p, batch, h, items, merges, workers)
        assert h.num_partials * 16 * 512 * 2 <= h.partial_lse_offset - h.partial_out_offset
        offs.add((h.items_offset, h.merges_offset, h.workers_offset, h.partial_out_offset,
                  h.partial_lse_offset, h.workspace_bytes))
    assert len(offs) == 1


def test_skewed_batch_splits_the_long_request_across_the_chip():
    batch = workloads.skewed_fp8()
    p = m.make_params(128, 64, kv_dtype=m.MLA_DTYPE_FP8_E4M3FN, num_cus=256)
    h, items, merges, workers = build(p, batch)
    check_invariants(p, batch, h, items, merges, workers)
    long_row = int(np.argmax(batch.seq_lens))
    long_chunks = [it for it in items if it.row == long_row]
    assert len(long_chunks) >= 128
    # no chunk is much longer than the balanced share of the whole batch
    total = int(batch.seq_lens.sum())
    assert max(it.kv_end - it.kv_begin for it in items) <= max(512, -(-total // 256)) + 4 * TILE


@pytest.mark.parametrize("name", ["v3", "v2_lite", "skewed_fp8"])
def test_workers_are_balanced(name):
    """The fill gives every worker nearly the same cost: the busiest is within
    one item's fixed cost plus a few tiles of the mean."""
    batch = getattr(workloads, name)()
    kv = m.MLA_DTYPE_FP8_E4M3FN if batch.cache_dtype != "bf16" else m.MLA_DTYPE_BF16
    p = m.make_params(batch.num_heads, batch.page_size, kv_dtype=kv, num_cus=256)
    h, items, merges, workers = build(p, batch)
    check_invariants(p, batch, h, items, merges, workers)
    cost = item_cost(batch.num_heads)
    loads = worker_loads(items, workers, cost)
    mean = sum(loads) / len(loads)
    assert max(loads) <= mean + cost + 8, (max(loads), mean)


@pytest.mark.parametrize("name,max_idle", [("v2_lite", 1), ("skewed_fp8", 3), ("v3", 1)])
def test_capacity_leaves_few_workers_idle(name, max_idle):
    """No worker's load exceeds the plan's capacity, and the capacity sits
    close enough to the mean load that at most a few workers get no item
    (two-tile pieces are taken where they lower the capacity; with whole
    item-cost pieces the 16-head batch left 12 workers idle)."""
    batch = getattr(workloads, name)()
    kv = m.MLA_DTYPE_FP8_E4M3FN if batch.cache_dtype != "bf16" else m.MLA_DTYPE_BF16
    p = m.make_params(batch.num_heads, batch.page_size, kv_dtype=kv, num_cus=256)
    h, items, merges, workers = build(p, batch)
    loads = worker_loads(items, workers, item_cost(batch.num_heads))
    assert max(loads) * TILE <= h.chunk_tokens
    idle = sum(1 for w in range(h.num_workers) if workers[w + 1] == workers[w])
    assert idle <= max_idle, idle


def test_empty_requests_get_an_empty_item():
    batch = workloads.random_decode_batch(3, [0, 5, 0], 16, 4)
    p = m.make_params(16, 4, num_cus=256)
    h, items, merges, workers = build(p, batch)
    check_invariants(p, batch, h, items, merges, workers)
    empty = [it for it in items if it.kv_begin == it.kv_end]
    assert sorted(it.row for it in empty) == [0, 2]


def test_graph_safe_plans_list_every_worker_and_record_their_counts():
    """Graph-safe plans: all G workers listed (the launch always has them), the
    flags recorded, the wide-merge count in the header; the planner rejects
    unknown flags and the decode call rejects a plan built with other flags."""
    for H, G in ((128, 64), (16, 64)):
        p = m.make_params(H, 64, num_cus=64, flags=m.MLA_DECODE_GRAPH_SAFE, max_rows=8)
        batch = workloads.random_decode_batch(77, [20000, 300, 5, 2600], num_heads=H, page_size=64)
        pb, _ = m.mla_decode_workspace_size(p, batch.batch, batch.num_rows)
        plan = np.zeros(pb, dtype=np.uint8)
        assert m.mla_decode_plan(p, batch.batch, None, batch.kv_indptr, batch.kv_last_page_len,
                                 plan, pb) == m.MLA_OK
        h, items, merges, workers = m.read_plan(plan)
        assert h.flags == m.MLA_DECODE_GRAPH_SAFE and h.num_workers == G
        assert len(workers) == G + 1 and workers[-1] == h.num_items
        assert h.num_wide_merges == sum(1 for mi in merges if mi.num_partials >= 16) >= 1
        # The fixed merge grids of a graph-safe launch bound the plan's counts.
        assert h.num_merges <= G - 1 and h.num_wide_merges <= -(-(G - 1) // 15)
    bad = m.make_params(16, 1, num_cus=8, flags=2)
    plan = np.zeros(1 << 16, dtype=np.uint8)
    assert m.mla_decode_plan(bad, 1, None, np.array([0, 3], np.int32), None, plan,
                             plan.size) == m.MLA_ERR_UNSUPPORTED


def test_graph_safe_plans_share_one_layout():
    """Captured launches keep the workspace addresses of the plan they were
    captured with, so every graph-safe plan of the same params must put its
    items, merges, worker table and partials at the same offsets, whatever
    its batch: those of the bound for max_rows rows."""
    fields = ("items_offset", "merges_offset", "workers_offset", "plan_bytes", "partial_out_offset",
              "partial_lse_offset", "workspace_bytes")
    for H in (16, 128):
        p = m.make_params(H, 16, num_cus=16, flags=m.MLA_DECODE_GRAPH_SAFE, max_rows=6)
        pb, wb = m.mla_decode_workspace_size(p, 6, 6)
        seen = []
        for k, lens in enumerate([[3000, 40, 1, 700, 64, 2000], [10, 5000, 300, 0, 33, 17], [900, 900, 1], [5]]):
            batch = workloads.random_decode_batch(50 + k, lens, num_heads=H, page_size=16)
            plan = np.zeros(pb, dtype=np.uint8)
            assert m.mla_decode_plan(p, batch.batch, None, batch.kv_indptr, batch.kv_last_page_len,
                                     plan, pb) == m.MLA_OK
            h = m.read_plan(plan)[0]
            seen.append((h.num_items, h.num_merges, tuple(getattr(h, f) for f in fields)))
        assert len({s[0:2] for s in seen}) > 1, "the batches should differ in items or merges"
        assert len({s[2] for s in seen}) == 1, seen
        assert seen[0][2][3] == pb and seen[0][2][6] == wb
        # More rows than max_rows: rejected; graph-safe without max_rows: rejected.
        big = workloads.random_decode_batch(60, [5] * 7, num_heads=H, page_size=16)
        plan = np.zeros(1 << 22, dtype=np.uint8)
        assert m.mla_decode_plan(p, 7, None, big.kv_indptr, big.kv_last_page_len, plan,
                                 plan.size) == m.MLA_ERR_INVALID_ARG
        p0 = m.make_params(H, 16, num_cus=16, flags=m.MLA_DECODE_GRAPH_SAFE)
        assert m.mla_decode_plan(p0, 1, None, np.array([0, 1], np.int32), None, plan,
                                 plan.size) == m.MLA_ERR_INVALID_ARG


def test_tree_verify_plans_keep_every_suffix_slot_in_the_last_chunk():
    """suffix_tokens S: each row is planned S tokens longer, no chunk boundary
    falls inside its last S tokens (so only its last chunk, flagged, reads the
    suffix table), and the planner takes S only for H = 128 at page size 1."""
    S = 8
    p = m.make_params(128, 1, num_cus=16, suffix_tokens=S)
    lens = [2048, 2048, 1, 0, 5000, 300, 31, 33]
    batch = workloads.random_decode_batch(70, lens, num_heads=128, page_size=1, rows_per_request=3)
    pb, _ = m.mla_decode_workspace_size(p, batch.batch, batch.num_rows)
    plan = np.zeros(pb, dtype=np.uint8)
    assert m.mla_decode_plan(p, batch.batch, batch.qo_indptr, batch.kv_indptr, batch.kv_last_page_len,
                             plan, pb) == m.MLA_OK
    h, items, merges, _ = m.read_plan(plan)
    assert h.suffix_tokens == S and h.num_merges > 0
    row_len = np.repeat(np.asarray(lens), 3)
    for it in items:
        Lp = int(row_len[it.row])
        if it.flags & m.MLA_ITEM_LAST_CHUNK:
            assert it.kv_end == Lp + S and it.kv_begin <= Lp
        else:
            assert it.kv_end <= Lp
    for bad in (m.make_params(16, 1, suffix_tokens=S), m.make_params(128, 16, suffix_tokens=S),
                m.make_params(128, 1, suffix_tokens=257)):
        assert m.mla_decode_plan(bad, 1, None, np.array([0, 4], np.int32), None, plan,
                                 plan.size) == m.MLA_ERR_UNSUPPORTED
