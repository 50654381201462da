"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI, and compare with the oracle at the stated
tolerances (bf16 output: max-abs 2e-2 and relative L2 5e-3; fp32 mode:
max-abs 1e-5; lse: max-abs 1e-3)."""
import sys

import numpy as np
import torch

TOL_BF16_MAX_ABS = 2e-2
TOL_BF16_REL_L2 = 5e-3
TOL_FP32_MAX_ABS = 1e-5
TOL_LSE_MAX_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a GPU")
    return torch.device("cuda:0")


def bf16_to_device(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def batch_to_device(batch, dev):
    qn = bf16_to_device(batch.q_nope, dev)
    qr = bf16_to_device(batch.q_rope, dev)
    if batch.cache_dtype == "bf16":
        cache = bf16_to_device(batch.cache, dev)
    else:
        cache = torch.from_numpy(np.ascontiguousarray(batch.cache)).to(dev)
    idx = torch.from_numpy(np.ascontiguousarray(batch.kv_indices, dtype=np.int32)).to(dev)
    return qn, qr, cache, idx


def run_decode(batch, dev, out_dtype="bf16", max_splits=0, kv_lens=None, num_cus=0,
               q_pair=None, shared_rows=False):
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    qn, qr, cache, idx = batch_to_device(batch, dev)
    if q_pair is not None:
        qn, qr = q_pair
    dec = PagedMlaDecoder(batch.num_heads, batch.page_size, max_batch=batch.batch,
                          max_rows=batch.num_rows, kv_dtype=batch.cache_dtype, out_dtype=out_dtype,
                          num_cus=num_cus, max_splits=max_splits, device=dev, shared_rows=shared_rows)
    rows_per_req = np.diff(batch.qo_indptr)
    qo = None if np.all(rows_per_req == 1) else batch.qo_indptr
    dec.plan(batch.kv_indptr, batch.kv_last_page_len, qo)
    kl = None if kv_lens is None else torch.from_numpy(np.asarray(kv_lens, np.int32)).to(dev)
    out, lse = dec.run(qn, qr, cache, idx, batch.sm_scale, batch.kv_scale, kl)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), dec


def compare(out, lse, out_ref, lse_ref, fp32, what=""):
    assert out.shape == out_ref.shape and lse.shape == lse_ref.shape
    assert np.isfinite(out).all(), f"{what}: non-finite output (a canary was read?)"
    err = np.abs(out - out_ref)
    max_abs = float(err.max()) if err.size else 0.0
    ref_norm = float(np.linalg.norm(out_ref))
    rel = float(np.linalg.norm(out - out_ref) / ref_norm) if ref_norm > 0 else max_abs
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf_ref), f"{what}: -inf lse pattern differs"
    fin = ~ninf_ref
    lse_err = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} lse_max_abs={lse_err:.3e}")
    if fp32:
        assert max_abs <= TOL_FP32_MAX_ABS, f"{what}: fp32 max_abs {max_abs}"
    else:
        assert max_abs <= TOL_BF16_MAX_ABS, f"{what}: max_abs {max_abs}"
        assert rel <= TOL_BF16_REL_L2, f"{what}: rel_l2 {rel}"
    assert lse_err <= TOL_LSE_MAX_ABS, f"{what}: lse {lse_err}"
    return max_abs, rel, lse_err
