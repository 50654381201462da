"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (default plan over all of the device's compute units): the whole batch
runs on the GPU and every row is checked against the oracle. The tree-verify cascade runs end to end:
compaction, prefix decode, suffix decode with device-side lengths, LSE merge,
against the oracle's attention over the prefix plus the visible drafts."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_mla_decode_amd import _binding as binding
from gpu_util import batch_to_device, compare, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def run_full(batch, dev, out_dtype):
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    qn, qr, cache, idx = batch_to_device(batch, dev)
    dec = PagedMlaDecoder(batch.num_heads, batch.page_size, max_batch=batch.batch,
                          max_rows=batch.num_rows, kv_dtype=batch.cache_dtype, out_dtype=out_dtype,
                          device=dev)
    dec.plan(batch.kv_indptr, batch.kv_last_page_len)
    plan = binding.read_plan(dec.plan_h)
    out, lse = dec.run(qn, qr, cache, idx, batch.sm_scale, batch.kv_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), plan


_ORACLE = {}


def oracle_full(name, batch):
    """The oracle over the whole batch (every row and head), computed once per
    workload: a few seconds on the host's cores."""
    if name not in _ORACLE:
        _ORACLE.clear()  # one workload's reference at a time (V3: 67 MB)
        _ORACLE[name] = oracle.decode_batch(batch)
    return _ORACLE[name]


@pytest.mark.parametrize("name,out_dtype", [
    ("v2_lite", "bf16"),
    ("v3", "bf16"),
    ("v3", "fp32"),
    ("skewed_fp8", "bf16"),
])
def test_config_all_rows(dev, name, out_dtype):
    """Every row and head of the full-size workload against the oracle, and
    the whole output finite (no canary read anywhere)."""
    batch = getattr(workloads, name)()
    say(f"config {name} out={out_dtype}: B={batch.batch} H={batch.num_heads} ps={batch.page_size} "
        f"tokens={int(batch.seq_lens.sum())}")
    out, lse, (h, items, merges, workers) = run_full(batch, dev, out_dtype)
    say(f"  plan: workers={h.num_workers} items={h.num_items} merges={h.num_merges} "
        f"capacity={h.chunk_tokens} tokens")
    assert np.isfinite(out).all() and not np.isnan(lse).any()
    ref_out, ref_lse = oracle_full(name, batch)
    split_rows = len({mi.row for mi in merges})
    say(f"  all {batch.num_rows} rows, {split_rows} of them split")
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", f"{name} all rows")
    if name in ("v3", "skewed_fp8"):
        assert split_rows > 0, "the workload must exercise split-KV rows"


@pytest.mark.parametrize("mode", ["merge_states", "suffix_merge", "single_pass"])
def test_tree_verify_cascade(dev, mode):
    from paged_mla_decode_amd.decoder import PagedMlaDecoder, merge_states, tree_suffix_compact
    tv = workloads.tree_verify()
    pre = tv.prefix
    W, D = tv.width, tv.max_tree_depth
    B = pre.batch
    N = pre.num_rows
    say(f"tree cascade ({mode}): B={B} W={W} rows={N} "
        f"prefix={int(pre.seq_lens[0])} depth<={D}")
    qn, qr, cache, idx = batch_to_device(pre, dev)

    # 1. stable compaction of the suffix tables (one launch)
    mask_d = torch.from_numpy(tv.tree_mask).to(dev)
    r2t_d = torch.from_numpy(tv.req_to_token).to(dev)
    pl_d = torch.from_numpy(tv.prefix_lens).to(dev)
    table, seqlens = tree_suffix_compact(mask_d, r2t_d, pl_d, W)
    seq_h = seqlens.cpu().numpy()
    assert np.array_equal(seq_h, tv.tree_mask.sum(axis=1)), "seqlens = visible drafts per row"
    assert seq_h.max() <= D, "depth bound: truncation to max_tree_depth drops nothing"

    if mode == "single_pass":
        # 2-4. one pass: each row over its prefix and then its visible drafts
        d1 = PagedMlaDecoder(pre.num_heads, 1, max_batch=B, max_rows=N, device=dev, suffix_tokens=D)
        d1.plan(pre.kv_indptr, pre.kv_last_page_len, pre.qo_indptr)
        out, lse = d1.run_tree_verify(qn, qr, cache, idx, table, seqlens, pre.sm_scale)
    # 2. prefix: every draft row attends to its request's prefix
    dp = PagedMlaDecoder(pre.num_heads, 1, max_batch=B, max_rows=N, device=dev)
    dp.plan(pre.kv_indptr, pre.kv_last_page_len, pre.qo_indptr)
    out_p, lse_p = dp.run(qn, qr, cache, idx, pre.sm_scale)

    # 3. suffix: row r attends to the first D entries of its compacted table,
    #    clipped on the device to its visible count
    ds = PagedMlaDecoder(pre.num_heads, 1, max_batch=N, max_rows=N, device=dev)
    ds.plan(np.arange(N + 1, dtype=np.int32) * D, np.ones(N, dtype=np.int32))
    suffix_idx = table[:, :D].contiguous().view(-1)
    if mode == "single_pass":
        # The two-pass cascade on the same rows must agree with the single pass
        # to bf16 rounding (checked below against the oracle as well).
        out_s, lse_s = ds.run(qn, qr, cache, suffix_idx, pre.sm_scale, kv_lens=seqlens)
        out2, lse2 = merge_states(out_p, lse_p, out_s, lse_s)
        torch.cuda.synchronize()
        d2 = (out.float() - out2.float()).abs().max().item()
        dl = (lse - lse2).abs().max().item()
        say(f"  single pass vs two-pass cascade: max_abs={d2:.3e} lse={dl:.3e}")
        assert d2 <= 2e-2 and dl <= 1e-3
    elif mode == "suffix_merge":
        # 3+4. the suffix attention merged with the prefix state in the same call, in place
        out, lse = ds.run_suffix_merge(qn, qr, cache, suffix_idx, pre.sm_scale, out_p, lse_p,
                                       kv_lens=seqlens, out=out_p, lse=lse_p)
    else:
        out_s, lse_s = ds.run(qn, qr, cache, suffix_idx, pre.sm_scale, kv_lens=seqlens)
        # 4. LSE merge of the two states
        out, lse = merge_states(out_p, lse_p, out_s, lse_s)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)

    # Oracle: attention of each sampled row over prefix + its visible drafts.
    rng = np.random.Generator(np.random.PCG64(12))
    rows = np.unique(np.concatenate([
        np.arange(0, N, W),                                     # every root row
        np.argsort(-tv.tree_mask.sum(axis=1), kind="stable")[:6],  # deepest rows
        rng.choice(N, size=10, replace=False)]))
    kv_indptr = [0]
    kv_indices = []
    for r in rows:
        req, plen = int(r) // W, int(tv.prefix_lens[int(r) // W])
        vis = np.nonzero(tv.tree_mask[r])[0]
        slots = np.concatenate([tv.req_to_token[req, :plen], tv.req_to_token[req, plen + vis]])
        kv_indices.append(slots)
        kv_indptr.append(kv_indptr[-1] + len(slots))
    ref_out, ref_lse = oracle.mla_decode(
        pre.q_nope[rows], pre.q_rope[rows], pre.cache, np.asarray(kv_indptr, np.int32),
        np.concatenate(kv_indices).astype(np.int32), 1, pre.sm_scale,
        kv_last_page_len=np.ones(len(rows), np.int32))
    say(f"  checking {len(rows)} rows")
    compare(out[rows], lse[rows], ref_out, ref_lse, False, "tree cascade")
