"""Parity of the HIP LSE merge and the tree-suffix stable compaction with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [512, 8, 1032])
def test_merge_states(dev, dtype, D):
    from paged_mla_decode_amd.decoder import merge_states
    rng = np.random.default_rng(D)
    n = 777
    va = rng.standard_normal((n, D)).astype(np.float32)
    vb = rng.standard_normal((n, D)).astype(np.float32)
    sa = (rng.standard_normal(n) * 5).astype(np.float32)
    sb = (rng.standard_normal(n) * 5).astype(np.float32)
    sa[::7] = -np.inf
    sb[::11] = -np.inf  # row 0 and every 77th: both empty
    va[::7] = 0
    vb[::11] = 0
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    ta, tb = torch.from_numpy(va).to(dev, tdt), torch.from_numpy(vb).to(dev, tdt)
    # the oracle merges exactly what the device sees
    va_d, vb_d = ta.double().cpu().numpy(), tb.double().cpu().numpy()
    ref_v, ref_s = oracle.merge_states(va_d, sa.astype(np.float64), vb_d, sb.astype(np.float64))
    say(f"merge dtype={dtype} D={D}")
    out, s = merge_states(ta, torch.from_numpy(sa).to(dev), tb, torch.from_numpy(sb).to(dev))
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    s = s.double().cpu().numpy()
    assert np.array_equal(np.isneginf(s), np.isneginf(ref_s))
    fin = np.isfinite(ref_s)
    assert np.abs(s[fin] - ref_s[fin]).max() < 1e-5
    tol = 1e-5 if dtype == "fp32" else 2e-2
    assert np.abs(o - ref_v).max() <= tol * max(1.0, np.abs(ref_v).max())
    # in place (out aliases a)
    merge_states(ta, torch.from_numpy(sa).to(dev), tb, torch.from_numpy(sb).to(dev), out=ta)
    torch.cuda.synchronize()
    assert np.array_equal(ta.double().cpu().numpy(), o)


def _compact_on_device(dev, mask, r2t, prefix, width, rows, n_actual):
    from paged_mla_decode_amd.decoder import tree_suffix_compact
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(r2t, dtype=np.int32)).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(prefix, dtype=np.int32)).to(dev)
    table, seqlens = tree_suffix_compact(m, t, p, width, num_rows=rows, num_actual_rows=n_actual)
    torch.cuda.synchronize()
    return table.cpu().numpy(), seqlens.cpu().numpy()


def test_compaction_tree_workload_bit_exact(dev):
    tv = workloads.tree_verify()
    n = tv.tree_mask.shape[0]
    say("compaction tree workload")
    ref_t, ref_s = oracle.tree_suffix_compact(tv.tree_mask, tv.req_to_token, tv.prefix_lens,
                                              tv.width, rows=n + 13, num_actual_rows=n)
    t, s = _compact_on_device(dev, tv.tree_mask, tv.req_to_token, tv.prefix_lens, tv.width, n + 13, n)
    assert np.array_equal(t, ref_t) and np.array_equal(s, ref_s)
    assert s[:n].max() <= tv.max_tree_depth


@pytest.mark.parametrize("width", [1, 3, 8, 10])
def test_compaction_all_masks_bit_exact(dev, width):
    masks = ((np.arange(2 ** width)[:, None] >> np.arange(width)[None, :]) & 1).astype(np.uint8)
    rows = masks.shape[0]
    nreq = -(-rows // width)
    rng = np.random.default_rng(width)
    prefix = rng.integers(0, 9, size=nreq).astype(np.int32)
    r2t = rng.integers(0, 1 << 30, size=(nreq, width + 9)).astype(np.int32)
    say(f"compaction all masks W={width}")
    ref_t, ref_s = oracle.tree_suffix_compact(masks, r2t, prefix, width)
    t, s = _compact_on_device(dev, masks, r2t, prefix, width, rows, rows)
    assert np.array_equal(t, ref_t) and np.array_equal(s, ref_s)


@pytest.mark.parametrize("width", [64, 65, 130, 1024])
def test_compaction_wide_rows(dev, width):
    rng = np.random.default_rng(width)
    rows = 3 * width
    mask = (rng.random((rows, width)) < 0.3).astype(np.uint8)
    nreq = 3
    prefix = rng.integers(0, 100, size=nreq).astype(np.int32)
    r2t = rng.integers(0, 1 << 30, size=(nreq, width + 100)).astype(np.int32)
    say(f"compaction W={width}")
    ref_t, ref_s = oracle.tree_suffix_compact(mask, r2t, prefix, width)
    t, s = _compact_on_device(dev, mask, r2t, prefix, width, rows, rows)
    assert np.array_equal(t, ref_t) and np.array_equal(s, ref_s)
