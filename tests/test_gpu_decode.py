"""Parity of the HIP decode path (through the C ABI) with the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import compare, require_gpu, run_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_tiny(dev, out_dtype):
    batch = workloads.tiny()
    say(f"tiny out={out_dtype}")
    out, lse, dec = run_decode(batch, dev, out_dtype)
    assert dec.variant == f"mla_decode<hw16,hs2,kv_bf16,out_{out_dtype}>"
    ref_out, ref_lse = oracle.decode_batch(batch)
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", "tiny")


LENS = [1, 31, 32, 33, 100, 257, 64, 600]


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("ps", [1, 16, 64])
def test_shapes(dev, H, ps):
    batch = workloads.random_decode_batch(100 + H + ps, LENS, num_heads=H, page_size=ps)
    say(f"shapes H={H} ps={ps}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    for splits in (1, 0, 4):
        out, lse, dec = run_decode(batch, dev, "bf16", max_splits=splits, num_cus=8)
        h = dec.header()
        if splits == 1:
            assert h.num_merges == 0
        compare(out, lse, ref_out, ref_lse, False, f"H={H} ps={ps} splits={splits} merges={h.num_merges}")


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("ps", [3, 48])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_odd_page_sizes(dev, H, ps, kv):
    """Page sizes that are not powers of two take the kernels' division and
    remainder branch of the address generation (token -> page, in-page row);
    tiles then straddle pages at arbitrary tokens."""
    batch = workloads.random_decode_batch(300 + H + ps, LENS, num_heads=H, page_size=ps, cache_dtype=kv)
    say(f"odd page size H={H} ps={ps} kv={kv}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    for splits in (1, 0):
        out, lse, dec = run_decode(batch, dev, "bf16", max_splits=splits, num_cus=8)
        h = dec.header()
        compare(out, lse, ref_out, ref_lse, False, f"H={H} ps={ps} kv={kv} merges={h.num_merges}")


@pytest.mark.parametrize("H", [16, 128])
def test_fp32_mode_with_splits(dev, H):
    batch = workloads.random_decode_batch(7 + H, [5, 300, 1000, 77], num_heads=H, page_size=16)
    say(f"fp32 H={H}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, "fp32", num_cus=4)
    assert dec.header().num_merges > 0
    compare(out, lse, ref_out, ref_lse, True, f"fp32 H={H}")


@pytest.mark.parametrize("H", [16, 32, 128])
@pytest.mark.parametrize("ps", [1, 64])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_fp8_cache(dev, H, ps, out_dtype):
    batch = workloads.random_decode_batch(11 + H + ps, [3, 64, 129, 500], num_heads=H, page_size=ps,
                                          cache_dtype="fp8_e4m3fn")
    say(f"fp8 H={H} ps={ps} out={out_dtype}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, out_dtype, num_cus=4)
    assert "kv_fp8" in dec.variant
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", f"fp8 H={H} ps={ps}")


@pytest.mark.parametrize("ps", [16, 64])
def test_kv_lens_clips_on_device(dev, ps):
    """Device lengths shorter than the plan's (a truncated cascade suffix): whole
    chunks past the clip, chunks cut inside a tile, and a request clipped to 0.
    At 64 tokens per page the 128-head kernel takes the page-uniform tiles."""
    batch = workloads.random_decode_batch(21 + ps, [40, 200, 333, 64], num_heads=128, page_size=ps)
    clip = np.array([17, 200, 100, 0], np.int32)
    say(f"kv_lens clip ps={ps}")
    out, lse, _ = run_decode(batch, dev, "bf16", kv_lens=clip, num_cus=4)
    # oracle over the clipped lengths: same pages, fewer tokens
    L = clip
    npages = (L + ps - 1) // ps
    kv_indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    kv_indices = np.concatenate([batch.kv_indices[batch.kv_indptr[b]:batch.kv_indptr[b] + npages[b]]
                                 for b in range(batch.batch)]).astype(np.int32)
    last = np.where(L > 0, L - ps * (npages - 1), 1).astype(np.int32)
    ref_out, ref_lse = oracle.mla_decode(batch.q_nope, batch.q_rope, batch.cache, kv_indptr,
                                         kv_indices, ps, batch.sm_scale, kv_last_page_len=last)
    compare(out, lse, ref_out, ref_lse, False, f"kv_lens ps={ps}")


def test_empty_requests(dev):
    batch = workloads.random_decode_batch(22, [0, 45, 0, 1], num_heads=16, page_size=8)
    say("empty requests")
    ref_out, ref_lse = oracle.decode_batch(batch)
    for splits in (1, 0):
        out, lse, _ = run_decode(batch, dev, "bf16", max_splits=splits, num_cus=2)
        compare(out, lse, ref_out, ref_lse, False, f"empty splits={splits}")
        assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("H", [16, 128])
def test_extreme_score_spread_takes_the_exact_rerun(dev, H):
    """A token far past the first tile with a score ~150 (log2) above the rest:
    the fixed softmax reference would overflow, so the kernel recomputes."""
    batch = workloads.random_decode_batch(23, [300, 90], num_heads=H, page_size=1)
    rows = workloads.token_rows(batch.kv_indptr, batch.kv_indices, batch.seq_lens, 1)
    hot = workloads.bf16_bits_to_f32(batch.cache.reshape(-1, 576)[rows[200]])
    qn = workloads.bf16_bits_to_f32(batch.q_nope).copy()
    qn[0, :, :] = hot[:512] * 10.0
    batch.q_nope = workloads.f32_to_bf16_bits(qn)
    say(f"extreme spread H={H}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    assert ref_lse[0].min() - math.log(2) * 64 > 0  # the spread is really that large
    out, lse, _ = run_decode(batch, dev, "fp32", max_splits=1)
    compare(out, lse, ref_out, ref_lse, True, "extreme fp32")
    out, lse, _ = run_decode(batch, dev, "bf16", max_splits=0, num_cus=2)
    compare(out, lse, ref_out, ref_lse, False, "extreme bf16 split")


def test_concatenated_query_through_strides(dev):
    batch = workloads.random_decode_batch(24, [70, 5, 130], num_heads=64, page_size=4)
    say("strided q")
    from gpu_util import bf16_to_device
    q_cat = np.concatenate([batch.q_nope, batch.q_rope], axis=-1)  # [N, H, 576]
    qd = bf16_to_device(q_cat, dev)
    out, lse, _ = run_decode(batch, dev, "bf16", q_pair=(qd[..., :512], qd[..., 512:]))
    ref_out, ref_lse = oracle.decode_batch(batch)
    compare(out, lse, ref_out, ref_lse, False, "strided q")


def test_multiple_query_rows_per_request(dev):
    batch = workloads.random_decode_batch(25, [50, 300, 17], num_heads=128, page_size=1,
                                          rows_per_request=4)
    say("qo rows")
    out, lse, _ = run_decode(batch, dev, "bf16", num_cus=4)
    ref_out, ref_lse = oracle.decode_batch(batch)
    compare(out, lse, ref_out, ref_lse, False, "qo rows")


def test_deterministic(dev):
    batch = workloads.random_decode_batch(26, [700, 1500, 90], num_heads=128, page_size=64)
    say("determinism")
    a, la, _ = run_decode(batch, dev, "bf16", num_cus=8)
    b, lb, _ = run_decode(batch, dev, "bf16", num_cus=8)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3fn"])
def test_one_worker_runs_every_item(dev, cache_dtype):
    """Plans for one and two compute units: a persistent workgroup runs many
    items in turn (empty requests, partial tiles, a piece of a split row and,
    for the bf16 cache, a row whose score spread forces the exact rerun), so
    every piece of per-item state must start fresh."""
    lens = [0, 1, 31, 32, 33, 700, 0, 65, 2000, 300]
    batch = workloads.random_decode_batch(31, lens, num_heads=128, page_size=64, cache_dtype=cache_dtype)
    if cache_dtype == "bf16":
        # Request 9: one token far past the first tile scores ~150 (log2) above the rest.
        rows = workloads.token_rows(batch.kv_indptr, batch.kv_indices, batch.seq_lens, 64)
        hot = workloads.bf16_bits_to_f32(batch.cache.reshape(-1, 576)[rows[int(np.sum(batch.seq_lens[:9])) + 250]])
        qn = workloads.bf16_bits_to_f32(batch.q_nope).copy()
        qn[9, :, :] = hot[:512] * 10.0
        batch.q_nope = workloads.f32_to_bf16_bits(qn)
    say(f"one worker {cache_dtype}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    if cache_dtype == "bf16":
        assert ref_lse[9].min() - math.log(2) * 64 > 0  # the rerun path is taken
    # One compute unit: one worker runs all ten items. Two: the second worker runs
    # nine of them, the first of which is the tail piece of a split row.
    for cus in (1, 2):
        out, lse, dec = run_decode(batch, dev, "bf16", num_cus=cus, max_splits=3)
        h = dec.header()
        assert h.num_workers == cus and (cus == 1 or h.num_merges > 0)
        compare(out, lse, ref_out, ref_lse, False, f"{cus} worker(s) {cache_dtype}")


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_many_partials_take_the_wide_merge(dev, H, out_dtype):
    """A long request cut into dozens of pieces: its partials are merged by a
    workgroup per row and head, the short rows' by one wave per row and head,
    in the same merge launch."""
    batch = workloads.random_decode_batch(41 + H, [20000, 300, 5, 2600], num_heads=H, page_size=16)
    say(f"wide merge H={H} out={out_dtype}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, out_dtype, num_cus=64)
    assert dec.header().max_merge_partials >= 16
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", f"wide merge H={H} out={out_dtype}")


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("ps", [32, 128, 1024])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_large_page_sizes(dev, H, ps, kv):
    """Pages of one tile or larger (a 1024-token page holds 32 tiles): the shift
    branch of the address generation with many tiles per page, partial last
    pages, and requests shorter than one page. At 128 heads these take the
    page-uniform tile path (one page number per tile), 32 being its smallest page."""
    lens = [1, ps - 1, ps, ps + 1, 3 * ps + 17, 2000]
    batch = workloads.random_decode_batch(330 + H + ps, lens, num_heads=H, page_size=ps, cache_dtype=kv)
    say(f"large page size H={H} ps={ps} kv={kv}")
    ref_out, ref_lse = oracle.decode_batch(batch)
    for splits in (1, 0):
        out, lse, dec = run_decode(batch, dev, "bf16", max_splits=splits, num_cus=8)
        compare(out, lse, ref_out, ref_lse, False, f"H={H} ps={ps} kv={kv} merges={dec.header().num_merges}")
