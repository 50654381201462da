"""Seeded random small batches through the decode entry points against the
oracle: head counts, page sizes (powers of two and not), bf16 and fp8 caches,
bf16 and fp32 outputs, several query rows per request with and without shared
rows, CU counts and split caps drawn per case; the fused append (outputs, and
the cache bit for bit), the fused prefix merge (in place and not), the fp8
score and the single tree-verify pass on random batches of their own."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import compare, require_gpu, run_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("seed", range(48))
def test_random_batch_against_the_oracle(dev, seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.choice([0, 1, 5, 31, 32, 33, 200, 777, 1500, 3000], size=B)]
    ps = int(rng.choice([1, 3, 16, 64, 128]))
    H = int(rng.choice([16, 32, 64, 128]))
    kv = str(rng.choice(["bf16", "fp8_e4m3fn"]))
    out_dtype = str(rng.choice(["bf16", "fp32"]))
    rows = [int(x) for x in rng.integers(0, 5, size=B)] if rng.random() < 0.5 else 1
    shared = bool(rng.random() < 0.5)
    cus = int(rng.choice([1, 7, 32, 256]))
    splits = int(rng.choice([0, 0, 1, 3]))
    batch = workloads.random_decode_batch(2000 + seed, lens, num_heads=H, page_size=ps, cache_dtype=kv,
                                          rows_per_request=rows)
    what = (f"seed={seed} B={B} lens={lens} ps={ps} H={H} kv={kv} out={out_dtype} rows={rows} "
            f"shared={shared} cus={cus} splits={splits}")
    say(what)
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, out_dtype, max_splits=splits, num_cus=cus, shared_rows=shared)
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", what)


@pytest.mark.parametrize("seed", range(16))
def test_random_append_against_the_oracle(dev, seed):
    """mla_decode_append on random batches: outputs within the tolerances and
    the whole cache after the call bit for bit against write-then-decode."""
    from test_gpu_append import new_rows, run_append
    rng = np.random.Generator(np.random.PCG64(3000 + seed))
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.choice([1, 2, 31, 32, 33, 200, 1500, 3000], size=B)]
    ps = int(rng.choice([1, 3, 16, 64, 128]))
    H = int(rng.choice([16, 32, 64, 128]))
    kv = str(rng.choice(["bf16", "fp8_e4m3fn"]))
    out_dtype = str(rng.choice(["bf16", "fp32"]))
    cus = int(rng.choice([1, 7, 32, 256]))
    batch = workloads.random_decode_batch(4000 + seed, lens, num_heads=H, page_size=ps, cache_dtype=kv)
    c, r = new_rows(5000 + seed, B)
    what = f"append seed={seed} lens={lens} ps={ps} H={H} kv={kv} out={out_dtype} cus={cus}"
    say(what)
    ref_out, ref_lse, ref_cache = oracle.append_then_decode(
        batch.q_nope, batch.q_rope, batch.cache, batch.kv_indptr, batch.kv_indices,
        batch.kv_last_page_len, batch.page_size, batch.sm_scale, c, r, batch.kv_scale)
    out, lse, cache, _ = run_append(batch, dev, c, r, out_dtype=out_dtype, num_cus=cus)
    assert np.array_equal(cache, ref_cache), f"{what}: cache differs from write-then-decode"
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", what)


@pytest.mark.parametrize("seed", range(16))
def test_random_suffix_merge_against_the_oracle(dev, seed):
    """mla_decode_suffix_merge on random prefix / suffix splits (page size 1):
    the merged state equals the oracle's attention over the union."""
    import torch
    from test_gpu_cascade import split_csr
    from gpu_util import batch_to_device
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    rng = np.random.Generator(np.random.PCG64(6000 + seed))
    B = int(rng.integers(1, 7))
    prefix = [int(x) for x in rng.choice([0, 1, 5, 33, 300, 1500], size=B)]
    suffix = [int(x) for x in rng.choice([0, 1, 7, 32, 200, 1500], size=B)]
    H = int(rng.choice([16, 32, 64, 128]))
    out_dtype = str(rng.choice(["bf16", "fp32"]))
    inplace = bool(rng.random() < 0.5)
    cus = int(rng.choice([1, 7, 32, 256]))
    batch = workloads.random_decode_batch(7000 + seed, [p + s for p, s in zip(prefix, suffix)],
                                          num_heads=H, page_size=1)
    (pi, pidx, plast), (si, sidx, slast) = split_csr(batch, prefix)
    what = f"suffix merge seed={seed} prefix={prefix} suffix={suffix} H={H} out={out_dtype} inplace={inplace} cus={cus}"
    say(what)
    qn, qr, cache, _ = batch_to_device(batch, dev)
    dp = PagedMlaDecoder(H, 1, max_batch=B, out_dtype=out_dtype, num_cus=cus, device=dev)
    dp.plan(pi, plast)
    pidx_d = torch.from_numpy(pidx).to(dev) if len(pidx) else torch.zeros(1, dtype=torch.int32, device=dev)
    sidx_d = torch.from_numpy(sidx).to(dev) if len(sidx) else torch.zeros(1, dtype=torch.int32, device=dev)
    out_p, lse_p = dp.run(qn, qr, cache, pidx_d, batch.sm_scale)
    ds = PagedMlaDecoder(H, 1, max_batch=B, out_dtype=out_dtype, num_cus=cus, device=dev)
    ds.plan(si, slast)
    kw = dict(out=out_p, lse=lse_p) if inplace else {}
    out, lse = ds.run_suffix_merge(qn, qr, cache, sidx_d, batch.sm_scale, out_p, lse_p, **kw)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_batch(batch)
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_out, ref_lse, out_dtype == "fp32", what)


@pytest.mark.parametrize("seed", range(12))
def test_random_fp8_score_against_the_oracle(dev, seed):
    """MLA_DECODE_FP8_SCORE on random e4m3fn batches (128 heads, bf16 output,
    several rows per request at times): within the bound derived for the fp8
    matrix core and within the plain bf16 gates, against the oracle with the
    dequantised query."""
    from test_gpu_fp8_score import check, reference
    rng = np.random.Generator(np.random.PCG64(8000 + seed))
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.choice([0, 1, 5, 31, 32, 33, 200, 777, 1500, 3000], size=B)]
    ps = int(rng.choice([1, 3, 16, 64, 128]))
    rows = [int(x) for x in rng.integers(0, 4, size=B)] if rng.random() < 0.5 else 1
    if rows != 1 and sum(rows) == 0:
        rows[0] = 1
    cus = int(rng.choice([1, 7, 32, 256]))
    splits = int(rng.choice([0, 0, 1, 3]))
    batch = workloads.random_decode_batch(9000 + seed, lens, num_heads=128, page_size=ps,
                                          cache_dtype="fp8_e4m3fn", rows_per_request=rows)
    what = f"fp8 score seed={seed} lens={lens} ps={ps} rows={rows} cus={cus} splits={splits}"
    say(what)
    import torch
    from gpu_util import batch_to_device
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    qn, qr, cache, idx = batch_to_device(batch, dev)
    dec = PagedMlaDecoder(128, ps, max_batch=B, max_rows=max(1, batch.num_rows), kv_dtype="fp8_e4m3fn",
                          num_cus=cus, max_splits=splits, device=dev, fp8_score=True)
    qo = None if np.all(np.diff(batch.qo_indptr) == 1) else batch.qo_indptr
    dec.plan(batch.kv_indptr, batch.kv_last_page_len, qo)
    out, lse = dec.run(qn, qr, cache, idx, batch.sm_scale, batch.kv_scale)
    torch.cuda.synchronize()
    ref_out, ref_lse, D, M = reference(batch)
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
          ref_out, ref_lse, D, M, what)


@pytest.mark.parametrize("seed", range(8))
def test_random_tree_verify_against_the_oracle(dev, seed):
    """mla_decode_tree_verify on random prefixes, row counts, suffix caps and
    suffix tables: each row against the oracle over its request's prefix and
    then its visible suffix slots."""
    import torch
    from gpu_util import batch_to_device
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    rng = np.random.Generator(np.random.PCG64(10000 + seed))
    B = int(rng.integers(1, 5))
    prefix = [int(x) for x in rng.choice([1, 5, 33, 300, 2048], size=B)]
    rows = [int(x) for x in rng.integers(1, 6, size=B)]
    S = int(rng.choice([1, 8, 64, 256]))
    stride = S + int(rng.integers(0, 5))
    cus = int(rng.choice([1, 7, 32, 256]))
    batch = workloads.random_decode_batch(11000 + seed, prefix, num_heads=128, page_size=1, rows_per_request=rows)
    N = batch.num_rows
    counts = rng.integers(0, S + 1, size=N).astype(np.int32)
    valid = batch.kv_indices[:int(batch.kv_indptr[-1])]
    table = np.zeros((N, stride), np.int32)
    for r in range(N):
        table[r, :counts[r]] = rng.choice(valid, size=int(counts[r]), replace=True)
    what = f"tree verify seed={seed} prefix={prefix} rows={rows} S={S} counts={counts.tolist()} cus={cus}"
    say(what)
    qn, qr, cache, idx = batch_to_device(batch, dev)
    d = PagedMlaDecoder(128, 1, max_batch=B, max_rows=N, num_cus=cus, device=dev, suffix_tokens=S)
    d.plan(batch.kv_indptr, batch.kv_last_page_len, batch.qo_indptr)
    out, lse = d.run_tree_verify(qn, qr, cache, idx, torch.from_numpy(table).to(dev),
                                 torch.from_numpy(counts).to(dev), batch.sm_scale)
    torch.cuda.synchronize()
    row_req = np.repeat(np.arange(B), np.diff(batch.qo_indptr))
    indptr, indices = [0], []
    for r in range(N):
        b = row_req[r]
        slots = np.concatenate([batch.kv_indices[batch.kv_indptr[b]:batch.kv_indptr[b + 1]], table[r, :counts[r]]])
        indices.append(slots)
        indptr.append(indptr[-1] + len(slots))
    ref_out, ref_lse = oracle.mla_decode(batch.q_nope, batch.q_rope, batch.cache, np.asarray(indptr, np.int32),
                                         np.concatenate(indices).astype(np.int32), 1, batch.sm_scale,
                                         kv_last_page_len=np.ones(N, np.int32))
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_out, ref_lse, False, what)
