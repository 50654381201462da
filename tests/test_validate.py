"""Host checks of index arrays against the pool (mla_decode_validate_batch,
mla_tree_validate_inputs, mla_tree_validate_suffix), through the C ABI on the
CPU only: the decode calls read whatever pool rows the entries name, so a bad
entry is caught here and never reaches a device."""
import numpy as np
import pytest

import oracle
import workloads
from paged_mla_decode_amd import _binding as B


def batch_args(batch):
    return (batch.page_size, batch.batch, None, batch.kv_indptr, batch.kv_indices,
            batch.kv_last_page_len, batch.cache.shape[0])


@pytest.mark.parametrize("ps", [1, 3, 64])
def test_generated_batches_pass(ps):
    batch = workloads.random_decode_batch(5 + ps, [0, 1, 31, 200, 64], num_heads=16, page_size=ps)
    assert B.mla_decode_validate_batch(*batch_args(batch)) == (B.MLA_OK, -1)


def test_out_of_pool_entries_are_named():
    batch = workloads.random_decode_batch(7, [40, 300, 2], num_heads=16, page_size=16)
    pages = batch.cache.shape[0]
    for at, bad in [(0, -1), (3, pages), (len(batch.kv_indices) - 1, pages + 1000), (5, -(2 ** 31))]:
        idx = batch.kv_indices.copy()
        idx[at] = bad
        st, where = B.mla_decode_validate_batch(batch.page_size, batch.batch, None, batch.kv_indptr,
                                                idx, batch.kv_last_page_len, pages)
        assert (st, where) == (B.MLA_ERR_INVALID_ARG, at)
    # the last page of the pool is a page of it
    idx = batch.kv_indices.copy()
    idx[2] = pages - 1
    assert B.mla_decode_validate_batch(batch.page_size, batch.batch, None, batch.kv_indptr, idx,
                                       batch.kv_last_page_len, pages)[0] == B.MLA_OK
    # entries past kv_indptr[batch] are not part of the batch
    extra = np.concatenate([batch.kv_indices, np.array([-5, pages * 2], np.int32)])
    assert B.mla_decode_validate_batch(batch.page_size, batch.batch, None, batch.kv_indptr, extra,
                                       batch.kv_last_page_len, pages)[0] == B.MLA_OK


def test_malformed_csr_and_lengths():
    ip = np.array([0, 2, 5], np.int32)
    ix = np.arange(5, dtype=np.int32)
    last = np.array([4, 1], np.int32)
    ok = B.mla_decode_validate_batch(4, 2, None, ip, ix, last, 5)
    assert ok == (B.MLA_OK, -1)
    cases = [
        (4, 2, None, np.array([1, 2, 5], np.int32), ix, last, 5),        # does not start at 0
        (4, 2, None, np.array([0, 3, 2], np.int32), ix, last, 5),        # decreasing
        (4, 2, None, ip, ix, np.array([0, 1], np.int32), 5),              # last page empty
        (4, 2, None, ip, ix, np.array([4, 5], np.int32), 5),              # last page over ps
        (4, 2, np.array([0, 2, 1], np.int32), ip, ix, last, 5),           # qo_indptr decreasing
        (0, 2, None, ip, ix, last, 5),                                    # page size
        (4, 2, None, ip, None, last, 5),                                  # no indices
    ]
    for c in cases:
        assert B.mla_decode_validate_batch(*c)[0] == B.MLA_ERR_INVALID_ARG, c
    # a request without pages has length 0 whatever its last-page entry says
    ip0 = np.array([0, 0, 5], np.int32)
    assert B.mla_decode_validate_batch(4, 2, None, ip0, ix, np.array([0, 1], np.int32), 5)[0] == B.MLA_OK


def tree_case():
    tv = workloads.tree_verify(seed=40, batch=3, prefix_len=50, width=16, max_depth=4, pool_slots=512)
    return tv


def test_tree_inputs():
    tv = tree_case()
    r2t = np.ascontiguousarray(tv.req_to_token, np.int32)
    pool = tv.prefix.cache.shape[0]
    args = (r2t, r2t.shape[1], r2t.shape[0], tv.prefix_lens, tv.width, pool)
    assert B.mla_tree_validate_inputs(*args) == (B.MLA_OK, -1)
    bad = r2t.copy()
    at = 1 * r2t.shape[1] + int(tv.prefix_lens[1]) + 7  # a draft slot of request 1
    bad.reshape(-1)[at] = pool
    assert B.mla_tree_validate_inputs(bad, *args[1:]) == (B.MLA_ERR_INVALID_ARG, at)
    # prefix slots are not read by the compaction (kv_indices covers them)
    pre = r2t.copy()
    pre[0, 0] = -1
    assert B.mla_tree_validate_inputs(pre, *args[1:])[0] == B.MLA_OK
    # the draft columns must fit the row
    long = tv.prefix_lens.copy()
    long[2] = r2t.shape[1] - tv.width + 1
    assert B.mla_tree_validate_inputs(r2t, args[1], args[2], long, tv.width, pool)[0] == \
        B.MLA_ERR_INVALID_ARG


def test_tree_suffix_table():
    tv = tree_case()
    table, seqlens = oracle.tree_suffix_compact(tv.tree_mask, tv.req_to_token, tv.prefix_lens, tv.width)
    pool = tv.prefix.cache.shape[0]
    S = tv.max_tree_depth
    args = (table, table.shape[1], seqlens, table.shape[0], S, pool)
    assert B.mla_tree_validate_suffix(*args) == (B.MLA_OK, -1)
    # an entry past the row's visible count is never read
    t2 = table.copy()
    r = int(np.argmin(seqlens))
    t2[r, seqlens[r]] = -1
    assert B.mla_tree_validate_suffix(t2, *args[1:])[0] == B.MLA_OK
    # one inside it is
    t3 = table.copy()
    r = int(np.argmax(seqlens))
    t3[r, 0] = pool
    assert B.mla_tree_validate_suffix(t3, *args[1:]) == (B.MLA_ERR_INVALID_ARG, r * table.shape[1])
    # rows longer than the truncation read only S entries
    t4 = table.copy()
    s4 = seqlens.copy()
    s4[0] = S + 5
    t4[0, S:] = -7
    assert B.mla_tree_validate_suffix(t4, table.shape[1], s4, table.shape[0], S, pool)[0] == B.MLA_OK
    s5 = seqlens.copy()
    s5[1] = -1
    assert B.mla_tree_validate_suffix(table, table.shape[1], s5, table.shape[0], S, pool)[0] == \
        B.MLA_ERR_INVALID_ARG
