"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: the
absorption identity against decompressed multi-head attention, a library
attention routine, closed forms, invariances, split+merge equal to unsplit,
brute force, and the element decoders against torch over every code.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import ROW, SM_SCALE


# ---------------------------------------------------------------------------
# Element decoders
# ---------------------------------------------------------------------------

def test_bf16_decoder_matches_torch_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_double(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_double(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


# ---------------------------------------------------------------------------
# Helpers that gather tokens without going through the oracle
# ---------------------------------------------------------------------------

def _tokens(batch, b):
    """Cache rows (float64 [L, 576]) of request b, gathered by numpy."""
    L = int(batch.seq_lens[b])
    t = np.arange(L)
    pages = batch.kv_indices[batch.kv_indptr[b] + t // batch.page_size].astype(np.int64)
    rows = pages * batch.page_size + t % batch.page_size
    flat = batch.cache.reshape(-1, ROW)[rows]
    if batch.cache_dtype == "bf16":
        return workloads.bf16_bits_to_f32(flat).astype(np.float64)
    codes = torch.from_numpy(flat).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return codes * batch.kv_scale


def _q(batch):
    return (workloads.bf16_bits_to_f32(batch.q_nope).astype(np.float64),
            workloads.bf16_bits_to_f32(batch.q_rope).astype(np.float64))


# ---------------------------------------------------------------------------
# Absorption identity (SGLang v0.3 MLA page, self-test answer 2; sglang-jax MLA
# gap page, section 2.1): q . (W_UK c)^T = (q W_UK^T) . c^T, and W_UV moves to
# the output side. Checked against plain MHA with decompressed K and V.
# ---------------------------------------------------------------------------

def test_absorption_identity_against_decompressed_mha():
    batch = workloads.tiny()
    H, A, D = 16, 512, 128
    rng = np.random.Generator(np.random.PCG64(11))
    # Weights in the [A, N, H] layout of the MLAEinsum split (section 2.2 of the gap page).
    w_uk = rng.standard_normal((A, H, D)) / math.sqrt(A)
    w_uv = rng.standard_normal((A, H, D)) / math.sqrt(A)
    q_nope_heads = rng.standard_normal((batch.num_rows, H, D)) * 0.5
    _, q_rope = _q(batch)
    # Absorbed query: per head, q_nope (128) times W_UK^T -> 512; W_UV on the output.
    q_abs = oracle.absorb_query(q_nope_heads, w_uk)
    out_lat, lse = oracle.mla_decode(q_abs, q_rope, batch.cache, batch.kv_indptr, batch.kv_indices,
                                     1, SM_SCALE, kv_last_page_len=batch.kv_last_page_len)
    out_abs = oracle.project_output(out_lat, w_uv)

    for b in range(batch.batch):
        c = _tokens(batch, b)  # [L, 576]
        k_nope = np.einsum("ta,ahd->thd", c[:, :A], w_uk)  # decompressed keys
        v = np.einsum("ta,ahd->thd", c[:, :A], w_uv)  # decompressed values
        for h in range(H):
            s = (k_nope[:, h, :] @ q_nope_heads[b, h] + c[:, A:] @ q_rope[b, h]) * SM_SCALE
            m = s.max()
            p = np.exp(s - m)
            ref = (p / p.sum()) @ v[:, h, :]
            np.testing.assert_allclose(out_abs[b, h], ref, rtol=1e-10, atol=1e-12)
            assert abs(lse[b, h] - (m + math.log(p.sum()))) < 1e-10


# ---------------------------------------------------------------------------
# Library routine: after absorption MLA is multi-query attention with one
# shared 576-wide key head and a 512-wide value head (MLA paragraph of the
# attention-backends page). torch's SDPA in float64 on the CPU must agree.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("make", [
    lambda: workloads.tiny(),
    lambda: workloads.random_decode_batch(7, [1, 63, 64, 65, 200], num_heads=16, page_size=64),
    lambda: workloads.random_decode_batch(8, [5, 130], num_heads=32, page_size=16,
                                          cache_dtype="fp8_e4m3fn"),
])
def test_oracle_matches_sdpa_float64(make):
    batch = make()
    out, lse = oracle.decode_batch(batch)
    qn, qr = _q(batch)
    for b in range(batch.batch):
        c = torch.from_numpy(_tokens(batch, b))
        q = torch.from_numpy(np.concatenate([qn[b], qr[b]], axis=-1))  # [H, 576]
        H = q.shape[0]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, :, None, :], c[None, None].expand(1, H, -1, -1),
            c[None, None, :, :512].expand(1, H, -1, -1), scale=SM_SCALE)[0, :, 0]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-11, atol=1e-13)
        ref_lse = torch.logsumexp((q @ c.T) * SM_SCALE, dim=-1).numpy()
        np.testing.assert_allclose(lse[b], ref_lse, rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_single_token_returns_its_latent():
    batch = workloads.random_decode_batch(3, [1, 1, 1], num_heads=16, page_size=1)
    out, lse = oracle.decode_batch(batch)
    for b in range(3):
        c = _tokens(batch, b)
        for h in range(16):
            assert np.array_equal(out[b, h], c[0, :512])
    assert np.isfinite(lse).all()


def test_zero_query_gives_mean_and_log_length():
    batch = workloads.random_decode_batch(4, [3, 17, 64, 65], num_heads=16, page_size=16)
    q0 = np.zeros((batch.num_rows, 16, 512))
    r0 = np.zeros((batch.num_rows, 16, 64))
    out, lse = oracle.mla_decode(q0, r0, batch.cache, batch.kv_indptr, batch.kv_indices, 16,
                                 SM_SCALE, kv_last_page_len=batch.kv_last_page_len)
    for b in range(batch.batch):
        c = _tokens(batch, b)
        np.testing.assert_allclose(out[b], np.broadcast_to(c[:, :512].mean(0), (16, 512)),
                                   rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[b], math.log(len(c)), rtol=1e-14)


def test_constant_latent_gives_ones_so_softmax_rows_sum_to_one():
    batch = workloads.random_decode_batch(5, [9, 40], num_heads=16, page_size=1)
    cache = workloads.bf16_bits_to_f32(batch.cache).astype(np.float64)
    cache[..., :512] = 1.0
    cache[..., 512:] = np.nan_to_num(cache[..., 512:])
    out, _ = oracle.mla_decode(batch.q_nope, batch.q_rope, cache, batch.kv_indptr,
                               batch.kv_indices, 1, SM_SCALE)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_dominant_token_is_selected():
    batch = workloads.random_decode_batch(6, [12], num_heads=16, page_size=1)
    c = _tokens(batch, 0)
    # Query aligned with token 5's latent, scaled so that its score beats the rest by > 700.
    q = np.broadcast_to(c[5, :512] * 1e4, (1, 16, 512)).copy()
    out, lse = oracle.mla_decode(q, np.zeros((1, 16, 64)), batch.cache, batch.kv_indptr,
                                 batch.kv_indices, 1, SM_SCALE)
    np.testing.assert_array_equal(out[0, 3], c[5, :512])


def test_empty_request_gives_zero_and_minus_infinity():
    batch = workloads.random_decode_batch(9, [0, 5, 0], num_heads=16, page_size=4)
    out, lse = oracle.decode_batch(batch)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.isfinite(lse[1]).all()


# ---------------------------------------------------------------------------
# Invariances: pool placement and page size change addresses only.
# ---------------------------------------------------------------------------

def _repage(batch, page_size, seed):
    """The same logical tokens in a freshly permuted pool with another page size."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv_indptr, kv_indices, last = workloads.layout_from_lengths(
        batch.seq_lens, page_size, int(2 * sum(-(-int(L) // page_size) for L in batch.seq_lens) + 1),
        rng)
    new_rows = workloads.token_rows(kv_indptr, kv_indices, batch.seq_lens, page_size)
    old_rows = workloads.token_rows(batch.kv_indptr, batch.kv_indices, batch.seq_lens,
                                    batch.page_size)
    pool = np.full(((kv_indices.max() + 1) * page_size, ROW), workloads.BF16_NAN, np.uint16)
    pool[new_rows] = batch.cache.reshape(-1, ROW)[old_rows]
    return kv_indptr, kv_indices, last, pool.reshape(-1, page_size, ROW)


@pytest.mark.parametrize("new_ps", [1, 7, 64])
def test_placement_and_page_size_invariance_is_bit_exact(new_ps):
    batch = workloads.random_decode_batch(10, [1, 50, 64, 129], num_heads=16, page_size=16)
    out, lse = oracle.decode_batch(batch)
    kv_indptr, kv_indices, last, pool = _repage(batch, new_ps, seed=100 + new_ps)
    out2, lse2 = oracle.mla_decode(batch.q_nope, batch.q_rope, pool, kv_indptr, kv_indices,
                                   new_ps, SM_SCALE, kv_last_page_len=last)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------------------
# Split-KV (Flash-Decoding paragraph of the attention-backends page) and the
# LSE merge (PR 49477 analysis, introduction): unsplit == split + merge.
# ---------------------------------------------------------------------------

def _decode_range(batch, b, t0, t1):
    """Oracle over tokens [t0, t1) of request b (page size 1 view of the same rows)."""
    rows = workloads.token_rows(batch.kv_indptr, batch.kv_indices, batch.seq_lens,
                                batch.page_size)
    start = int(np.sum(batch.seq_lens[:b]))
    sel = rows[start + t0:start + t1].astype(np.int32)
    flat = batch.cache.reshape(-1, 1, ROW)
    q0, q1 = batch.qo_indptr[b], batch.qo_indptr[b + 1]
    return oracle.mla_decode(batch.q_nope[q0:q1], batch.q_rope[q0:q1], flat,
                             np.array([0, len(sel)], np.int32), sel, 1, SM_SCALE,
                             qo_indptr=np.array([0, q1 - q0], np.int32))


def test_split_then_merge_equals_unsplit():
    batch = workloads.random_decode_batch(12, [1, 37, 300], num_heads=16, page_size=8)
    out, lse = oracle.decode_batch(batch)
    rng = np.random.Generator(np.random.PCG64(13))
    for b in range(batch.batch):
        L = int(batch.seq_lens[b])
        cuts = np.sort(rng.integers(0, L + 1, size=4))
        bounds = [0, *cuts.tolist(), L]  # repeated cuts make empty chunks
        v, s = _decode_range(batch, b, bounds[0], bounds[1])
        for i in range(1, len(bounds) - 1):
            v2, s2 = _decode_range(batch, b, bounds[i], bounds[i + 1])
            v, s = oracle.merge_states(v, s, v2, s2)
        np.testing.assert_allclose(v, out[b:b + 1], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(s, lse[b:b + 1], rtol=1e-13, atol=1e-13)


def test_merge_with_empty_side_and_symmetry():
    rng = np.random.Generator(np.random.PCG64(14))
    v = rng.standard_normal((5, 8))
    s = rng.standard_normal(5)
    empty_v = np.zeros((5, 8))
    empty_s = np.full(5, -np.inf)
    v1, s1 = oracle.merge_states(v, s, empty_v, empty_s)
    assert np.array_equal(v1, v) and np.array_equal(s1, s)
    v2, s2 = oracle.merge_states(empty_v, empty_s, empty_v, empty_s)
    assert np.all(v2 == 0) and np.all(np.isneginf(s2))
    w = rng.standard_normal((5, 8))
    t = rng.standard_normal(5)
    a, sa = oracle.merge_states(v, s, w, t)
    b, sb = oracle.merge_states(w, t, v, s)
    np.testing.assert_allclose(a, b, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(sa, sb, rtol=1e-15)
    # Closed form for equal weights: the mean, and ln 2 added.
    m, sm = oracle.merge_states(v, s, w, s)
    np.testing.assert_allclose(m, (v + w) / 2, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(sm, s + math.log(2), rtol=1e-15)


# ---------------------------------------------------------------------------
# Stable compaction (PR 49477 analysis, section 1): the suffix table is a
# stable partition, visible slots first, both groups in order.
# ---------------------------------------------------------------------------

def _partition_by_hand(mask_row, slots):
    vis = [int(s) for m, s in zip(mask_row, slots) if m]
    hid = [int(s) for m, s in zip(mask_row, slots) if not m]
    return vis + hid


@pytest.mark.parametrize("width", [1, 2, 5, 8, 10])
def test_compaction_brute_force_all_masks(width):
    masks = ((np.arange(2 ** width)[:, None] >> np.arange(width)[None, :]) & 1).astype(np.uint8)
    rows = masks.shape[0]
    nreq = -(-rows // width)
    rng = np.random.Generator(np.random.PCG64(width))
    prefix = rng.integers(0, 5, size=nreq).astype(np.int32)
    r2t = rng.permutation(10 * (nreq * (width + 5))).astype(np.int32)[:nreq * (width + 5)]
    r2t = r2t.reshape(nreq, width + 5)
    table, seqlens = oracle.tree_suffix_compact(masks, r2t, prefix, width)
    for r in range(rows):
        req = r // width
        slots = r2t[req, prefix[req]:prefix[req] + width]
        assert table[r].tolist() == _partition_by_hand(masks[r], slots)
        assert seqlens[r] == int(masks[r].sum())
        assert sorted(table[r].tolist()) == sorted(slots.tolist())


def test_compaction_on_tree_workload_and_padding_rows():
    tv = workloads.tree_verify(batch=3, prefix_len=40, width=64, pool_slots=4096)
    rows_total = tv.tree_mask.shape[0] + 5  # five graph-padding rows
    table, seqlens = oracle.tree_suffix_compact(tv.tree_mask, tv.req_to_token, tv.prefix_lens,
                                                tv.width, rows=rows_total,
                                                num_actual_rows=tv.tree_mask.shape[0])
    n = tv.tree_mask.shape[0]
    assert np.all(table[n:] == 0) and np.all(seqlens[n:] == 0)
    for r in range(n):
        req, i = divmod(r, tv.width)
        assert seqlens[r] == tv.depth[req, i]  # ancestor chain incl. self = depth
        assert seqlens[r] <= tv.max_tree_depth
        slots = tv.req_to_token[req, tv.prefix_lens[req]:tv.prefix_lens[req] + tv.width]
        assert table[r].tolist() == _partition_by_hand(tv.tree_mask[r], slots)


# ---------------------------------------------------------------------------
# The projections by brute force on a tiny case (one multiply-add at a time),
# and the identity that ties them together: with W_UV = W_UK, projecting the
# absorbed query back gives q_nope times the head's Gram matrix W^T W.
# ---------------------------------------------------------------------------

def test_projections_brute_force_and_gram_identity():
    rng = np.random.Generator(np.random.PCG64(12))
    N, H, A, D = 3, 2, 6, 4
    q = rng.standard_normal((N, H, D))
    w = rng.standard_normal((A, H, D))
    x = rng.standard_normal((N, H, A))
    qa = oracle.absorb_query(q, w)
    o = oracle.project_output(x, w)
    for n in range(N):
        for h in range(H):
            for a in range(A):
                acc = 0.0
                for d in range(D):
                    acc += q[n, h, d] * w[a, h, d]
                assert abs(qa[n, h, a] - acc) < 1e-12
            for d in range(D):
                acc = 0.0
                for a in range(A):
                    acc += x[n, h, a] * w[a, h, d]
                assert abs(o[n, h, d] - acc) < 1e-12
    back = oracle.project_output(qa, w)
    for h in range(H):
        gram = w[:, h, :].T @ w[:, h, :]
        np.testing.assert_allclose(back[:, h, :], q[:, h, :] @ gram, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Fused KV append (sglang-jax MLA gap page, sections 2.4 and 3.1). The encoder
# against torch's float8_e4m3fn cast (a library routine, round to nearest
# even) on every tie between neighbouring codes, every code value and random
# values; the append against closed forms and an invariance.
# ---------------------------------------------------------------------------

def _torch_e4m3fn(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encoder_matches_torch_on_ties_codes_and_random_values():
    vals = oracle.e4m3fn_to_double(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # exact in float32: few significant bits
    rng = np.random.Generator(np.random.PCG64(21))
    rand = np.exp(rng.uniform(np.log(2.0 ** -13), np.log(448.0), size=200_000))
    x = np.concatenate([vals, mids, rand, [0.0, 448.0]]).astype(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.e4m3fn_encode(x), _torch_e4m3fn(x))
    # Ties go to the even code: the midpoint of 0x01 and 0x02 is 0x02, of 0x02 and 0x03 is 0x02.
    assert oracle.e4m3fn_encode(np.float32(1.5 * 2.0 ** -9)) == 0x02
    assert oracle.e4m3fn_encode(np.float32(2.5 * 2.0 ** -9)) == 0x02
    assert oracle.e4m3fn_encode(np.float32(-0.0)) == 0x80


def test_e4m3fn_encode_decode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.e4m3fn_encode(oracle.e4m3fn_to_double(codes))
    # 0x80 (-0.0) decodes to -0.0 and comes back as 0x80.
    assert np.array_equal(back, codes)


def _last_rows(batch):
    """Latent and rope bits of each request's last token, gathered by numpy."""
    c, r = [], []
    for b in range(batch.batch):
        t = int(batch.seq_lens[b]) - 1
        page = batch.kv_indices[batch.kv_indptr[b] + t // batch.page_size]
        row = batch.cache[page, t % batch.page_size]
        c.append(row[:512])
        r.append(row[512:])
    return np.stack(c), np.stack(r)


def _append(batch, c_new, k_pe_new):
    return oracle.append_then_decode(batch.q_nope, batch.q_rope, batch.cache, batch.kv_indptr,
                                     batch.kv_indices, batch.kv_last_page_len, batch.page_size,
                                     batch.sm_scale, c_new, k_pe_new, batch.kv_scale)


def test_append_of_the_stored_row_changes_nothing():
    batch = workloads.random_decode_batch(31, [1, 5, 64, 65, 130], num_heads=16, page_size=16)
    c, r = _last_rows(batch)
    out, lse, cache = _append(batch, c, r)
    ref_out, ref_lse = oracle.decode_batch(batch)
    assert np.array_equal(cache, batch.cache)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3fn"])
def test_append_single_token_requests_return_the_new_row(cache_dtype):
    """L = 1: the softmax has one token, so out is the new latent as stored and
    lse its score. Only the new rows change in the cache."""
    batch = workloads.random_decode_batch(32, [1, 1, 1], num_heads=16, page_size=4,
                                          cache_dtype=cache_dtype)
    rng = np.random.Generator(np.random.PCG64(33))
    c = workloads.f32_to_bf16_bits(rng.standard_normal((3, 512), dtype=np.float32))
    r = workloads.f32_to_bf16_bits(rng.standard_normal((3, 64), dtype=np.float32))
    c[0, 0] = workloads.f32_to_bf16_bits(np.array([1e4], np.float32))[0]  # clamped to 448 in fp8
    out, lse, cache = _append(batch, c, r)
    row = np.concatenate([c, r], axis=1)
    vals = oracle.bf16_to_double(row)
    if cache_dtype == "fp8_e4m3fn":
        s = np.float32(batch.kv_scale)
        codes = _torch_e4m3fn(np.clip(vals.astype(np.float32) / s, -448, 448))
        vals = oracle.e4m3fn_to_double(codes) * batch.kv_scale
        assert codes[0, 0] == 0x7E
    qn, qr = _q(batch)
    for b in range(3):
        page = batch.kv_indices[batch.kv_indptr[b]]
        stored = cache[page, 0]
        expect = row[b] if cache_dtype == "bf16" else codes[b]
        assert np.array_equal(stored, expect)
        np.testing.assert_allclose(out[b], np.broadcast_to(vals[b, :512], (16, 512)), rtol=0, atol=1e-12)
        score = (qn[b] @ vals[b, :512] + qr[b] @ vals[b, 512:]) * SM_SCALE
        np.testing.assert_allclose(lse[b], score, rtol=1e-12, atol=1e-12)
    changed = np.nonzero((cache != batch.cache).any(axis=-1).ravel())[0]
    assert set(changed) <= {int(batch.kv_indices[batch.kv_indptr[b]]) * 4 for b in range(3)}


# ---------------------------------------------------------------------------
# Query quantisation of the optional fp8 score. Pinned against the definition's
# properties (minimal power-of-two exponent), torch's float8_e4m3fn cast of the
# scaled values, worked values and the e4m3fn error bound.
# ---------------------------------------------------------------------------

def _bf16(x):
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _quant_inputs(seed, N=6, H=5):
    rng = np.random.Generator(np.random.PCG64(seed))
    # Heads of very different magnitudes, one head of zeros, one exactly on a boundary.
    mag = np.exp2(rng.uniform(-20, 20, size=(N, H, 1)))
    q = rng.standard_normal((N, H, 576)) * mag
    q[0, 0] = 0.0
    q[1, 1] = 0.0
    q[1, 1, 7] = 448.0 * 2.0 ** 5           # amax exactly 448 * 2^5
    q[2, 2] = rng.standard_normal(576)
    q[2, 2, 3] = -448.0 * 2.0 ** -3 * (1 + 2.0 ** -7)  # just above 448 * 2^-3 (a bf16 value)
    bits = _bf16(q)
    return bits[..., :512], bits[..., 512:]


def test_query_quant_exponent_is_the_smallest_that_fits():
    qn, qr = _quant_inputs(41)
    _, _, e, _, _ = oracle.quantize_query_e4m3fn(qn, qr)
    q = np.concatenate([oracle.bf16_to_double(qn), oracle.bf16_to_double(qr)], axis=-1)
    amax = np.abs(q).max(axis=-1)
    nz = amax > 0
    assert (np.ldexp(amax[nz], -e[nz]) <= 448.0).all()
    assert (np.ldexp(amax[nz], -(e[nz] - 1)) > 448.0).all()
    assert e[0, 0] == 0 and e[1, 1] == 5 and e[2, 2] == -2


def test_query_quant_codes_match_torch_cast_of_scaled_values():
    qn, qr = _quant_inputs(42)
    cn, cr, e, hn, hr = oracle.quantize_query_e4m3fn(qn, qr)
    q = np.concatenate([oracle.bf16_to_double(qn), oracle.bf16_to_double(qr)], axis=-1)
    scaled = np.ldexp(q, -e[..., None].astype(np.int64))
    # Scaled bf16 values have 8 significant bits: exact in float32.
    assert np.array_equal(scaled.astype(np.float32).astype(np.float64), scaled)
    ref = _torch_e4m3fn(scaled.astype(np.float32))
    assert np.array_equal(np.concatenate([cn, cr], axis=-1), ref)
    back = torch.from_numpy(ref).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.concatenate([hn, hr], axis=-1), np.ldexp(back, e[..., None]))


def test_query_quant_worked_values():
    q = np.zeros((1, 3, 576))
    q[0, 0, :4] = [448.0, -1.0, 0.30078125, 0.0]  # 0.30078125: the bf16 value nearest 0.3
    q[0, 1, 0] = 1000.0                            # e = 2: 1000/4 = 250 fits, 1000/2 = 500 does not
    bits = _bf16(q)
    cn, _, e, hn, _ = oracle.quantize_query_e4m3fn(bits[..., :512], bits[..., 512:])
    assert list(e[0]) == [0, 2, 0]
    # 448 = 1.75 * 2^8: code 0x7E; -1: 0xB8; 0.30078125 lies between 0.28125 (0x29)
    # and 0.3125 (0x2A), nearer the latter.
    assert list(cn[0, 0, :4]) == [0x7E, 0xB8, 0x2A, 0x00]
    # 250 lies between 240 (0x77) and 256 (0x78), nearer 256: q_hat = 256 * 4.
    assert cn[0, 1, 0] == 0x78 and hn[0, 1, 0] == 1024.0
    assert (cn[0, 2] == 0).all() and (hn[0, 2] == 0).all()


def test_query_quant_error_within_half_a_step():
    qn, qr = _quant_inputs(43, N=16, H=8)
    _, _, e, hn, hr = oracle.quantize_query_e4m3fn(qn, qr)
    q = np.concatenate([oracle.bf16_to_double(qn), oracle.bf16_to_double(qr)], axis=-1)
    q_hat = np.concatenate([hn, hr], axis=-1)
    # e4m3fn has 3 fraction bits: half a step is 2^-4 of a normal value, and
    # half the subnormal step 2^-9 below 2^-6; both scale by 2^e.
    bound = np.maximum(2.0 ** -4 * np.abs(q), np.ldexp(2.0 ** -10, e[..., None]))
    assert (np.abs(q_hat - q) <= bound).all()
