"""mla_decode_noalloc (the library's own static device scratch instead of a
workspace) through the C ABI: two calls in a row on one GPU, the second with
a smaller batch, each equal bit for bit to mla_decode on the same plan and
inputs, and within the tolerances of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import batch_to_device, compare, require_gpu, say
from paged_mla_decode_amd import _binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def plan_host(p, batch):
    pb, wb = B.mla_decode_workspace_size(p, batch.batch, batch.num_rows)
    plan = np.zeros(pb, np.uint8)
    st = B.mla_decode_plan(p, batch.batch, None, batch.kv_indptr, batch.kv_last_page_len, plan, pb)
    assert st == B.MLA_OK, B.mla_status_string(st)
    return plan, wb


def run_both(dev, H, ps, lens, seed, kv="bf16"):
    batch = workloads.random_decode_batch(seed, lens, num_heads=H, page_size=ps, cache_dtype=kv)
    qn, qr, cache, idx = batch_to_device(batch, dev)
    kvd = B.MLA_DTYPE_FP8_E4M3FN if kv != "bf16" else B.MLA_DTYPE_BF16
    p = B.make_params(H, ps, kv_dtype=kvd, num_cus=16)
    plan, wb = plan_host(p, batch)
    h = B.read_plan(plan)[0]
    N = batch.num_rows
    stream = torch.cuda.current_stream().cuda_stream

    # The existing entry point: the plan copied into a workspace of its own.
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    st = B.mla_decode_plan(p, batch.batch, None, batch.kv_indptr, batch.kv_last_page_len, plan,
                           plan.nbytes, ws, wb, stream)
    assert st == B.MLA_OK
    ref_out = torch.empty((N, H, 512), dtype=torch.bfloat16, device=dev)
    ref_lse = torch.empty((N, H), dtype=torch.float32, device=dev)
    st = B.mla_decode(p, plan, ws, wb, qn, qn.stride(0), qn.stride(1), qr, qr.stride(0), qr.stride(1),
                      cache, batch.kv_scale, idx, None, batch.sm_scale, ref_out, ref_lse, stream)
    assert st == B.MLA_OK, B.mla_status_string(st)

    # The allocation-free one on the same host plan.
    out = torch.full((N, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((N, H), float("nan"), dtype=torch.float32, device=dev)
    st = B.mla_decode_noalloc(p, plan, qn, qn.stride(0), qn.stride(1), qr, qr.stride(0), qr.stride(1),
                              cache, batch.kv_scale, idx, None, batch.sm_scale, out, lse, stream)
    assert st == B.MLA_OK, B.mla_status_string(st)
    torch.cuda.synchronize()
    say(f"  noalloc H={H} ps={ps} kv={kv} rows={N}: items={h.num_items} merges={h.num_merges} "
        f"workspace={h.workspace_bytes} B")
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "noalloc differs from mla_decode"
    ref_o, ref_l = oracle.decode_batch(batch)
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_o, ref_l, False, f"noalloc H={H} vs oracle")
    return h


@pytest.mark.parametrize("H,ps,kv", [(128, 64, "bf16"), (16, 1, "bf16"), (128, 16, "fp8_e4m3fn")])
def test_noalloc_matches_mla_decode_twice(dev, H, ps, kv):
    say(f"noalloc H={H} ps={ps} kv={kv}: a batch, then a smaller one")
    h1 = run_both(dev, H, ps, [3000, 40, 700, 2000, 1, 64, 900, 5], 500 + H, kv)
    h2 = run_both(dev, H, ps, [333, 2, 1200], 600 + H, kv)
    assert h1.num_merges > 0 and h2.num_rows < h1.num_rows
