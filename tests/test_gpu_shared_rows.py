"""MLA_DECODE_SHARED_ROWS against the oracle: several query rows of a request
planned into one work item (up to 64 / H rows at 16 and 32 heads), each tile
loaded once for all of them. Every row still attends to all of its request's
tokens, so the oracle is the plain one over qo_indptr rows."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import compare, require_gpu, run_decode, say

pytestmark = pytest.mark.gpu

ROWS = [0, 4, 1, 9, 2, 3, 5]  # per request: none, a full unit, one, several units, partial units
LENS = [300, 1000, 0, 77, 2049, 1, 640]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("H", [16, 32])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_ragged_rows(dev, H, kv, out_dtype):
    batch = workloads.random_decode_batch(41, LENS, num_heads=H, page_size=16, cache_dtype=kv,
                                          rows_per_request=ROWS)
    say(f"shared rows H={H} kv={kv} out={out_dtype}: {batch.num_rows} rows")
    ref_out, ref_lse = oracle.decode_batch(batch)
    for cus, splits in ((256, 0), (8, 0), (1, 0), (256, 1)):
        out, lse, dec = run_decode(batch, dev, out_dtype, max_splits=splits, num_cus=cus, shared_rows=True)
        assert "hw16,hs4" in dec.variant
        compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", f"cus={cus} splits={splits}")


def test_rows_that_fill_units_exactly(dev):
    """Four rows per request at 16 heads: one unit per request, so every tile is
    read once per launch (the streaming load hint applies); long rows split."""
    batch = workloads.random_decode_batch(42, [5000, 3000, 64, 31], num_heads=16, page_size=1,
                                          rows_per_request=4)
    say("rows4 H=16")
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, "bf16", num_cus=16, shared_rows=True)
    assert dec._header.tiles_read_once == 1 and dec._header.num_merges > 0
    compare(out, lse, ref_out, ref_lse, False, "rows4")


@pytest.mark.parametrize("H", [64, 128])
def test_flag_is_a_no_op_where_one_row_fills_an_item(dev, H):
    batch = workloads.random_decode_batch(43, [90, 700, 5], num_heads=H, page_size=8, rows_per_request=[2, 3, 1])
    say(f"shared rows H={H}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, "bf16", num_cus=4, shared_rows=True)
    compare(out, lse, ref_out, ref_lse, False, f"H={H}")


def test_graph_safe_shared_rows(dev):
    """Graph-safe plans with shared rows: fixed merge grids sized for a partial per
    row of every split unit, checked against the oracle for two batches through
    one decoder (the second with fewer rows)."""
    import torch
    from gpu_util import batch_to_device
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    dec = PagedMlaDecoder(16, 1, max_batch=8, max_rows=40, device=dev, graph_safe=True, shared_rows=True,
                          num_cus=32)
    for seed, lens, rows in ((44, [4000, 100, 2500, 7], [4, 3, 9, 1]), (45, [50, 6000], [2, 5])):
        batch = workloads.random_decode_batch(seed, lens, num_heads=16, page_size=1, rows_per_request=rows)
        say(f"graph-safe shared rows {rows}")
        qn, qr, cache, idx = batch_to_device(batch, dev)
        dec.plan(batch.kv_indptr, batch.kv_last_page_len, batch.qo_indptr)
        out, lse = dec.run(qn, qr, cache, idx, batch.sm_scale, batch.kv_scale)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_batch(batch)
        n = batch.num_rows
        compare(out[:n].float().cpu().numpy().astype(np.float64), lse[:n].cpu().numpy().astype(np.float64),
                ref_out, ref_lse, False, f"graph-safe {rows}")


def test_v2_lite_four_rows_every_row(dev):
    """The V2-Lite-shaped batch with four query rows per request (256 rows), every
    row against the oracle."""
    batch = workloads.v2_lite(rows_per_request=4)
    say("v2_lite rows4 full size")
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, _ = run_decode(batch, dev, "bf16", shared_rows=True)
    assert np.isfinite(out).all()
    compare(out, lse, ref_out, ref_lse, False, "v2_lite rows4")
