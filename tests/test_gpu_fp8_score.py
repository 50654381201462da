"""The fp8 score (MLA_DECODE_FP8_SCORE) through the C ABI, against the oracle:
the quantised query bit for bit (codes and exponents as mla_decode leaves
them in its workspace), and the decode against the oracle's fp64 attention
with the dequantised query (``oracle.quantize_query_e4m3fn``).

Tolerance. The path differs from the bf16-score decode only in the score,
which the fp8 matrix core sums from exact products of e4m3fn values. Its
internal sums were measured within 2^-12 of the sum of the products'
magnitudes (one wave, random codes of every exponent), so each score, in
natural-log units, errs by at most D = 2^-12 * sm_scale * kv_scale *
max_t sum_k |code_q,k * 2^e * code_c,tk| for a row and head. Scores off by at
most D move the lse by at most D and every probability by a factor within
e^(+-2D), so each output element moves by at most (e^(2D) - 1) * max_t |v_t|.
Both terms are added to the bf16-output tolerances of the other decode tests,
which cover the rest of the arithmetic (identical to the fp8-cache path).
The 2^-12 figure is a measurement of the matrix core, not a derivation (its
internal summation order and rounding are not documented), so every check
also asserts the plain bf16 gates (max-abs 2e-2, relative L2 5e-3, lse 1e-3)
against the oracle with the dequantised query."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (TOL_BF16_MAX_ABS, TOL_BF16_REL_L2, TOL_LSE_MAX_ABS, batch_to_device,
                      require_gpu, say)

pytestmark = pytest.mark.gpu

MFMA_SUM_ERR = 2.0 ** -12


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def run_qf8(batch, dev, num_cus=0, graph_max_rows=None):
    """Decode with the fp8 score; returns out, lse (float64), the decoder and its plan header."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    qn, qr, cache, idx = batch_to_device(batch, dev)
    graph = graph_max_rows is not None
    dec = PagedMlaDecoder(batch.num_heads, batch.page_size, max_batch=batch.batch,
                          max_rows=graph_max_rows if graph else batch.num_rows,
                          kv_dtype=batch.cache_dtype, num_cus=num_cus, device=dev,
                          graph_safe=graph, fp8_score=True)
    qo = None if batch.num_rows == batch.batch else batch.qo_indptr
    h = dec.plan(batch.kv_indptr, batch.kv_last_page_len, qo)
    out, lse = dec.run(qn, qr, cache, idx, batch.sm_scale, batch.kv_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), dec, h


def score_bounds(batch, q_hat):
    """D [N, H] and M [N, 512] of the tolerance, from the dequantised operands
    (query rows qo_indptr[b] .. qo_indptr[b+1] attend to request b)."""
    flat = batch.cache.reshape(-1, 576)
    q_abs = np.abs(q_hat)
    D = np.zeros(q_hat.shape[:2])
    M = np.zeros((q_hat.shape[0], 512))
    for b in range(batch.batch):
        L = int(batch.seq_lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        rows = batch.kv_indices[batch.kv_indptr[b] + t // batch.page_size].astype(np.int64) * \
            batch.page_size + t % batch.page_size
        c = np.abs(oracle.e4m3fn_to_double(flat[rows])) * batch.kv_scale
        for n in range(int(batch.qo_indptr[b]), int(batch.qo_indptr[b + 1])):
            D[n] = (c @ q_abs[n].T).max(axis=0)
            M[n] = c[:, :512].max(axis=0)
    return MFMA_SUM_ERR * batch.sm_scale * D, M


def check(out, lse, ref_out, ref_lse, D, M, what):
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    fin = ~np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ~fin), f"{what}: -inf lse pattern differs"
    lse_err = np.abs(lse[fin] - ref_lse[fin])
    lse_tol = (TOL_LSE_MAX_ABS + D)[fin]
    slack = np.expm1(2 * D)[..., None] * M[:, None, :]
    err = np.abs(out - ref_out)
    # A batch of empty requests has an all-zero reference: compare absolutely.
    ref_norm = float(np.linalg.norm(ref_out))
    rel = float(np.linalg.norm(out - ref_out) / ref_norm) if ref_norm > 0 else float(err.max(initial=0.0))
    rel_tol = TOL_BF16_REL_L2 + (float(np.linalg.norm(np.broadcast_to(slack, out.shape)) / ref_norm)
                                 if ref_norm > 0 else 0.0)
    say(f"  {what}: max_abs={float(err.max(initial=0.0)):.3e} rel_l2={rel:.3e} (tol {rel_tol:.3e}) "
        f"lse_max_abs={float(lse_err.max(initial=0.0)):.3e} D max={float(D.max(initial=0.0)):.2e}")
    assert (lse_err <= lse_tol).all(), f"{what}: lse beyond bound"
    assert (err <= TOL_BF16_MAX_ABS + slack).all(), f"{what}: output beyond bound"
    assert rel <= rel_tol, f"{what}: rel_l2 {rel}"
    # The plain gates of the bf16 path hold as well: the derived slack above only
    # widens them by the fp8 matrix core's measured internal rounding.
    assert float(err.max(initial=0.0)) <= TOL_BF16_MAX_ABS, f"{what}: max_abs {float(err.max(initial=0.0))} (plain gate)"
    assert rel <= TOL_BF16_REL_L2, f"{what}: rel_l2 {rel} (plain gate)"
    assert float(lse_err.max(initial=0.0)) <= TOL_LSE_MAX_ABS, f"{what}: lse (plain gate)"


def reference(batch):
    _, _, _, hn, hr = oracle.quantize_query_e4m3fn(batch.q_nope, batch.q_rope)
    ref_out, ref_lse = oracle.mla_decode(hn, hr, batch.cache, batch.kv_indptr, batch.kv_indices,
                                         batch.page_size, batch.sm_scale,
                                         kv_last_page_len=batch.kv_last_page_len,
                                         qo_indptr=batch.qo_indptr, kv_scale=batch.kv_scale)
    D, M = score_bounds(batch, np.concatenate([hn, hr], axis=-1))
    return ref_out, ref_lse, D, M


LENS = [1, 31, 32, 33, 300, 2000]


def test_quantised_query_bit_exact(dev):
    batch = workloads.random_decode_batch(950, LENS, num_heads=128, page_size=64,
                                          cache_dtype="fp8_e4m3fn")
    q = np.concatenate([workloads.bf16_bits_to_f32(batch.q_nope),
                        workloads.bf16_bits_to_f32(batch.q_rope)], axis=-1)
    q[0, 0] = 0.0            # a head of zeros: e = 0, all codes 0
    q[0, 1] *= 2.0 ** 20     # large and small magnitudes: e far from 0
    q[0, 2] *= 2.0 ** -20
    q[1, 3, 100] = 448.0 * 4  # amax exactly 448 * 2^2
    bits = workloads.f32_to_bf16_bits(q)
    batch.q_nope, batch.q_rope = np.ascontiguousarray(bits[..., :512]), np.ascontiguousarray(bits[..., 512:])
    say("fp8 score: quantised query in the workspace")
    _, _, dec, h = run_qf8(batch, dev, num_cus=8)
    ws = dec.workspace.cpu().numpy()
    N, H = batch.num_rows, 128
    codes = ws[h.query_codes_offset:h.query_codes_offset + N * H * 576].reshape(N, H, 576)
    exps = ws[h.query_exp_offset:h.query_exp_offset + N * H * 4].view(np.int32).reshape(N, H)
    cn, cr, e, _, _ = oracle.quantize_query_e4m3fn(batch.q_nope, batch.q_rope)
    assert np.array_equal(exps, e), np.argwhere(exps != e)[:5]
    ref = np.concatenate([cn, cr], axis=-1)
    bad = np.argwhere(codes != ref)
    assert bad.size == 0, [(tuple(i), hex(codes[tuple(i)]), hex(ref[tuple(i)])) for i in bad[:5]]
    assert e[0, 0] == 0 and e[1, 3] == 2


@pytest.mark.parametrize("ps", [1, 32, 64])
@pytest.mark.parametrize("num_cus", [4, 0])
def test_fp8_score_parity(dev, ps, num_cus):
    batch = workloads.random_decode_batch(960 + ps + num_cus, LENS, num_heads=128, page_size=ps,
                                          cache_dtype="fp8_e4m3fn")
    say(f"fp8 score ps={ps} num_cus={num_cus}")
    out, lse, _, h = run_qf8(batch, dev, num_cus=num_cus)
    if num_cus == 4:
        assert h.num_merges > 0  # the long rows are split
    ref_out, ref_lse, D, M = reference(batch)
    check(out, lse, ref_out, ref_lse, D, M, f"fp8 score ps={ps} num_cus={num_cus}")


def test_fp8_score_several_rows_per_request(dev):
    """Three query rows per request (qo_indptr): each row has its own quantised
    query and exponents, and the rows of a request read the same tokens."""
    batch = workloads.random_decode_batch(975, [40, 1500, 1, 333], num_heads=128, page_size=16,
                                          cache_dtype="fp8_e4m3fn", rows_per_request=3)
    say(f"fp8 score, {batch.num_rows} rows over {batch.batch} requests")
    out, lse, _, h = run_qf8(batch, dev, num_cus=8)
    assert h.num_rows == 12
    ref_out, ref_lse, D, M = reference(batch)
    check(out, lse, ref_out, ref_lse, D, M, "fp8 score qo_indptr")


def test_fp8_score_empty_requests(dev):
    """Requests without tokens: lse -inf and a zero output, beside ordinary rows."""
    batch = workloads.random_decode_batch(977, [0, 5, 0, 700, 0], num_heads=128, page_size=64,
                                          cache_dtype="fp8_e4m3fn")
    say("fp8 score with empty requests")
    out, lse, _, _ = run_qf8(batch, dev, num_cus=8)
    ref_out, ref_lse, D, M = reference(batch)
    empty = batch.seq_lens == 0
    assert np.isneginf(lse[empty]).all() and (out[empty] == 0).all()
    check(out, lse, ref_out, ref_lse, D, M, "fp8 score empty requests")


def test_fp8_score_graph_safe_plan_with_fewer_rows(dev):
    batch = workloads.random_decode_batch(971, [5, 700, 64], num_heads=128, page_size=64,
                                          cache_dtype="fp8_e4m3fn")
    say("fp8 score, graph-safe plan with max_rows 9 for 3 rows")
    out, lse, _, _ = run_qf8(batch, dev, num_cus=8, graph_max_rows=9)
    ref_out, ref_lse, D, M = reference(batch)
    check(out, lse, ref_out, ref_lse, D, M, "fp8 score graph-safe")


def test_fp8_score_skewed_batch_all_rows(dev):
    """The skewed fp8 workload at full size (a 131,072-token request split
    across the chip beside 31 short ones), every row against the oracle."""
    batch = workloads.skewed_fp8()
    say(f"fp8 score, skewed fp8: tokens={int(batch.seq_lens.sum())}")
    out, lse, _, h = run_qf8(batch, dev)
    ref_out, ref_lse, D, M = reference(batch)
    say(f"  plan: items={h.num_items} merges={h.num_merges}; all {batch.num_rows} rows")
    check(out, lse, ref_out, ref_lse, D, M, "fp8 score skewed, all rows")
