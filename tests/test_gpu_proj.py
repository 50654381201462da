"""Parity of the two projections of weight absorption (W_UK into the query,
W_UV on the output; SGLang v0.3 MLA page, weight absorption; sglang-jax MLA
gap page, sections 2.1-2.2) with the CPU oracle, through the C ABI.

Element bound: the products of two bf16 values are exact in fp32, the K-term
fp32 sum errs by at most about K*2^-24 times the sum of |terms| (2^-15 for
K = 512; twice that is allowed), and the one rounding to bf16 adds at most
2^-8 of the value. So every element must satisfy
    |gpu - ref| <= 2^-8 |ref| + 2^-14 sum_k |a_k b_k|.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16_to_device, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def f64(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_bound(got, ref, abs_terms, what):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * abs_terms
    worst = float((err / np.maximum(bound, 1e-30)).max()) if err.size else 0.0
    say(f"  {what}: max_abs={float(err.max()) if err.size else 0.0:.3e} worst/bound={worst:.3f}")
    assert np.isfinite(got).all(), what
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} elements beyond the bound"


# Ragged row counts: one row, a partial 32-row block, several blocks plus a tail.
ROWS = [1, 5, 32, 77]


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("N", ROWS)
def test_absorb_query(dev, H, N):
    from paged_mla_decode_amd import absorb_query
    p = workloads.projection_inputs(1000 + N + H, N, H)
    say(f"absorb H={H} N={N}")
    ref = oracle.absorb_query(f64(p.q), f64(p.w_uk))
    terms = oracle.absorb_query(np.abs(f64(p.q)), np.abs(f64(p.w_uk)))
    got = absorb_query(bf16_to_device(p.q, dev), bf16_to_device(p.w_uk, dev))
    torch.cuda.synchronize()
    check_bound(to_f64(got), ref, terms, f"absorb H={H} N={N}")


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("N", ROWS)
def test_project_output(dev, H, N):
    from paged_mla_decode_amd import project_output
    p = workloads.projection_inputs(2000 + N + H, N, H)
    say(f"project H={H} N={N}")
    ref = oracle.project_output(f64(p.x), f64(p.w_uv))
    terms = oracle.project_output(np.abs(f64(p.x)), np.abs(f64(p.w_uv)))
    # W_UV with the latent contiguous: store it [H, D, A] and view it (a, h, d).
    w_t = bf16_to_device(np.ascontiguousarray(p.w_uv.transpose(1, 2, 0)), dev)
    got = project_output(bf16_to_device(p.x, dev), w_t.permute(2, 0, 1))
    torch.cuda.synchronize()
    check_bound(to_f64(got), ref, terms, f"project H={H} N={N}")


def test_strided_views_in_and_out(dev):
    """Strides as a model lays the tensors out: the nope half of a [N, H, 192]
    query, W_UK stored [H, A, D], the absorbed query written into the first 512
    columns of a [N, H, 576] decode query (its rope part untouched), W_UV as the
    value rows of a kv_b_proj weight [H*(128+128), 512], and the output into
    rows padded by 64 elements (the padding untouched)."""
    from paged_mla_decode_amd import absorb_query, project_output
    N, H, D, A = 45, 32, 128, 512
    p = workloads.projection_inputs(77, N, H)
    say("strided views")
    q_full = torch.zeros((N, H, 192), dtype=torch.bfloat16, device=dev)
    q_full[:, :, :D] = bf16_to_device(p.q, dev)
    w_uk = bf16_to_device(np.ascontiguousarray(p.w_uk.transpose(1, 0, 2)), dev).permute(1, 0, 2)
    qbuf = torch.full((N, H, 576), 7.0, dtype=torch.bfloat16, device=dev)
    absorb_query(q_full[:, :, :D], w_uk, out=qbuf[:, :, :A])
    # kv_b_proj rows of head h: 128 key-nope rows, then 128 value rows, each A wide.
    kvb = torch.zeros((H, 2 * D, A), dtype=torch.bfloat16, device=dev)
    kvb[:, D:, :] = bf16_to_device(np.ascontiguousarray(p.w_uv.transpose(1, 2, 0)), dev)
    kvb = kvb.reshape(H * 2 * D, A)
    w_uv = kvb.view(H, 2 * D, A)[:, D:, :].permute(2, 0, 1)
    obuf = torch.full((N, H * D + 64), 3.0, dtype=torch.bfloat16, device=dev)
    o = obuf.as_strided((N, H, D), (H * D + 64, D, 1))
    project_output(bf16_to_device(p.x, dev), w_uv, out=o)
    torch.cuda.synchronize()
    check_bound(to_f64(qbuf[:, :, :A]), oracle.absorb_query(f64(p.q), f64(p.w_uk)),
                oracle.absorb_query(np.abs(f64(p.q)), np.abs(f64(p.w_uk))), "absorb strided")
    assert bool((qbuf[:, :, A:] == 7.0).all()), "absorb wrote into the rope columns"
    check_bound(to_f64(o), oracle.project_output(f64(p.x), f64(p.w_uv)),
                oracle.project_output(np.abs(f64(p.x)), np.abs(f64(p.w_uv))), "project strided")
    assert bool((obuf[:, H * D:] == 3.0).all()), "project wrote into the row padding"


def test_decode_shape_full_size(dev):
    """The decode batch's own shape: 128 query rows of 128 heads, every element
    checked."""
    from paged_mla_decode_amd import absorb_query, project_output
    N, H = 128, 128
    p = workloads.projection_inputs(5, N, H)
    say("full size N=128 H=128")
    got = absorb_query(bf16_to_device(p.q, dev), bf16_to_device(p.w_uk, dev))
    w_t = bf16_to_device(np.ascontiguousarray(p.w_uv.transpose(1, 2, 0)), dev)
    o = project_output(bf16_to_device(p.x, dev), w_t.permute(2, 0, 1))
    torch.cuda.synchronize()
    check_bound(to_f64(got), oracle.absorb_query(f64(p.q), f64(p.w_uk)),
                oracle.absorb_query(np.abs(f64(p.q)), np.abs(f64(p.w_uk))), "absorb full")
    check_bound(to_f64(o), oracle.project_output(f64(p.x), f64(p.w_uv)),
                oracle.project_output(np.abs(f64(p.x)), np.abs(f64(p.w_uv))), "project full")


@pytest.mark.parametrize("H", [16, 128])
def test_absorb_decode_project_chain(dev, H):
    """W_UK absorption, paged decode and the W_UV projection chained on the
    device, against the oracle's fp64 chain (itself pinned to attention over
    the decompressed keys and values). The device rounds the absorbed query and
    the latent output to bf16 on the way; a relative L2 error of 1e-2 covers
    three bf16 roundings (each about 2^-9 rms) with room."""
    from paged_mla_decode_amd import absorb_query, project_output
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    batch = workloads.random_decode_batch(300 + H, [1, 40, 300, 1000, 64, 7], num_heads=H,
                                          page_size=16)
    N = batch.num_rows
    p = workloads.projection_inputs(400 + H, N, H)
    say(f"chain H={H}")
    q_abs_ref = oracle.absorb_query(f64(p.q), f64(p.w_uk))
    out_ref, lse_ref = oracle.mla_decode(q_abs_ref, batch.q_rope, batch.cache, batch.kv_indptr,
                                         batch.kv_indices, batch.page_size, batch.sm_scale,
                                         kv_last_page_len=batch.kv_last_page_len)
    o_ref = oracle.project_output(out_ref, f64(p.w_uv))

    qbuf = torch.empty((N, H, 576), dtype=torch.bfloat16, device=dev)
    qbuf[:, :, 512:] = bf16_to_device(batch.q_rope, dev)
    absorb_query(bf16_to_device(p.q, dev), bf16_to_device(p.w_uk, dev), out=qbuf[:, :, :512])
    dec = PagedMlaDecoder(H, batch.page_size, max_batch=batch.batch, num_cus=16, device=dev)
    dec.plan(batch.kv_indptr, batch.kv_last_page_len)
    cache = bf16_to_device(batch.cache, dev)
    idx = torch.from_numpy(np.ascontiguousarray(batch.kv_indices, dtype=np.int32)).to(dev)
    out, lse = dec.run(qbuf[:, :, :512], qbuf[:, :, 512:], cache, idx, batch.sm_scale)
    w_t = bf16_to_device(np.ascontiguousarray(p.w_uv.transpose(1, 2, 0)), dev)
    o = project_output(out, w_t.permute(2, 0, 1))
    torch.cuda.synchronize()
    o = to_f64(o)
    rel = float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))
    lse_err = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    say(f"  chain H={H}: rel_l2={rel:.3e} lse_max_abs={lse_err:.3e}")
    assert np.isfinite(o).all()
    assert rel <= 1e-2, rel
    assert lse_err <= 1e-2, lse_err
