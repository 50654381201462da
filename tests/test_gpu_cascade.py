"""mla_decode_suffix_merge: attention over a suffix merged by LSE with a given
prefix state in the same call (the fused suffix-attention + merge of the
PR 49477 analysis, section 3). Checked against the oracle's attention over
the union of the prefix and suffix tokens, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import batch_to_device, compare, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


# (prefix, suffix) tokens per request: empty suffix, empty prefix, both empty,
# a suffix long enough to be split across workers, ragged tails.
PREFIX = [5, 0, 0, 300, 40, 2000, 1]
SUFFIX = [0, 7, 0, 1500, 33, 64, 1]


def split_csr(batch, first):
    """Page lists of the first `first[b]` tokens and of the rest (page size 1)."""
    pi, ps_, si, ss = [0], [], [0], []
    for b in range(batch.batch):
        idx = batch.kv_indices[batch.kv_indptr[b]:batch.kv_indptr[b + 1]]
        pi.append(pi[-1] + first[b])
        ps_.append(idx[:first[b]])
        si.append(si[-1] + len(idx) - first[b])
        ss.append(idx[first[b]:])
    last = lambda ind: np.array([1 if ind[i + 1] > ind[i] else 0 for i in range(len(ind) - 1)], np.int32)
    return ((np.array(pi, np.int32), np.concatenate(ps_).astype(np.int32), last(pi)),
            (np.array(si, np.int32), np.concatenate(ss).astype(np.int32), last(si)))


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
def test_suffix_merge_equals_attention_over_the_union(dev, H, out_dtype, inplace):
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    lens = [p + s for p, s in zip(PREFIX, SUFFIX)]
    batch = workloads.random_decode_batch(1100 + H, lens, num_heads=H, page_size=1)
    (pi, pidx, plast), (si, sidx, slast) = split_csr(batch, PREFIX)
    say(f"suffix merge H={H} out={out_dtype} inplace={inplace}")
    qn, qr, cache, _ = batch_to_device(batch, dev)
    dp = PagedMlaDecoder(H, 1, max_batch=batch.batch, out_dtype=out_dtype, num_cus=8, device=dev)
    dp.plan(pi, plast)
    out_p, lse_p = dp.run(qn, qr, cache, torch.from_numpy(pidx).to(dev), batch.sm_scale)
    ds = PagedMlaDecoder(H, 1, max_batch=batch.batch, out_dtype=out_dtype, num_cus=8, device=dev)
    ds.plan(si, slast)
    assert ds.header().num_merges > 0  # the long suffix takes the merge kernel's prefix fold
    kw = dict(out=out_p, lse=lse_p) if inplace else {}
    out, lse = ds.run_suffix_merge(qn, qr, cache, torch.from_numpy(sidx).to(dev), batch.sm_scale,
                                   out_p, lse_p, **kw)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_batch(batch)  # attention over prefix + suffix tokens
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_out, ref_lse, out_dtype == "fp32", f"suffix merge H={H} {out_dtype}")


def test_suffix_merge_validates_aliasing(dev):
    from paged_mla_decode_amd import _binding as B
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    batch = workloads.random_decode_batch(1200, [3, 4], num_heads=16, page_size=1)
    qn, qr, cache, idx = batch_to_device(batch, dev)
    d = PagedMlaDecoder(16, 1, max_batch=2, device=dev)
    d.plan(batch.kv_indptr, batch.kv_last_page_len)
    po = torch.zeros((2, 16, 512), dtype=torch.bfloat16, device=dev)
    pl = torch.zeros((2, 16), dtype=torch.float32, device=dev)
    big = torch.zeros((3, 16, 512), dtype=torch.bfloat16, device=dev)
    with pytest.raises(B.MlaError):  # out overlaps the prefix without being it
        d.run_suffix_merge(qn, qr, cache, idx, batch.sm_scale, big[:2], pl, out=big[1:])


def test_tree_verify_single_pass_at_the_suffix_maximum(dev):
    """mla_decode_tree_verify with suffix_tokens at its maximum (256): rows with
    0, 1, 31-33, 255 and 256 visible suffix slots (whole tiles of suffix, and a
    table row stride above S), each against the oracle over its request's
    prefix and then its suffix slots."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    S, stride = 256, 260
    counts = [0, 1, 31, 32, 33, 255, 256, 100]
    batch = workloads.random_decode_batch(61, [37, 700], num_heads=128, page_size=1, rows_per_request=4)
    N = batch.num_rows
    rng = np.random.Generator(np.random.PCG64(62))
    valid = batch.kv_indices[:int(batch.kv_indptr[-1])]  # pool rows that hold values
    table = np.zeros((N, stride), np.int32)
    for r in range(N):
        table[r, :counts[r]] = rng.choice(valid, size=counts[r], replace=True)
    qn, qr, cache, idx = batch_to_device(batch, dev)
    d = PagedMlaDecoder(128, 1, max_batch=batch.batch, max_rows=N, device=dev, suffix_tokens=S)
    d.plan(batch.kv_indptr, batch.kv_last_page_len, batch.qo_indptr)
    out, lse = d.run_tree_verify(qn, qr, cache, idx, torch.from_numpy(table).to(dev),
                                 torch.from_numpy(np.asarray(counts, np.int32)).to(dev), batch.sm_scale)
    torch.cuda.synchronize()
    row_req = np.repeat(np.arange(batch.batch), np.diff(batch.qo_indptr))
    indptr, indices = [0], []
    for r in range(N):
        b = row_req[r]
        slots = np.concatenate([batch.kv_indices[batch.kv_indptr[b]:batch.kv_indptr[b + 1]], table[r, :counts[r]]])
        indices.append(slots)
        indptr.append(indptr[-1] + len(slots))
    ref_out, ref_lse = oracle.mla_decode(batch.q_nope, batch.q_rope, batch.cache, np.asarray(indptr, np.int32),
                                         np.concatenate(indices).astype(np.int32), 1, batch.sm_scale,
                                         kv_last_page_len=np.ones(N, np.int32))
    say(f"tree verify at S={S}: suffix counts {counts}")
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_out, ref_lse, False, "tree verify S=256")
