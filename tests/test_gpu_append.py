"""Fused KV append (mla_decode_append) against the oracle's write-then-decode,
through the C ABI: outputs at the decode tolerances, and the whole cache after
the call bit-exact (the new rows, and every other byte unchanged).

Before each call the new tokens' rows hold NaN canaries, so a tile that read
a row before the append landed would poison its outputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16_to_device, compare, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def new_rows(seed, n):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = workloads.f32_to_bf16_bits(rng.standard_normal((n, 512), dtype=np.float32) * np.float32(0.5))
    r = workloads.f32_to_bf16_bits(rng.standard_normal((n, 64), dtype=np.float32) * np.float32(0.5))
    return c, r


def last_slots(batch):
    """(page, in-page row) of each request's last token."""
    out = []
    for b in range(batch.batch):
        t = int(batch.seq_lens[b]) - 1
        out.append((int(batch.kv_indices[batch.kv_indptr[b] + t // batch.page_size]), t % batch.page_size))
    return out


def run_append(batch, dev, c_new, k_pe_new, out_dtype="bf16", num_cus=8, kv_scale=None):
    """Device run with canaries in the new rows; returns out, lse, cache after (numpy)."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    cache_np = np.array(batch.cache, copy=True)
    canary = workloads.BF16_NAN if batch.cache_dtype == "bf16" else workloads.E4M3FN_NAN
    for page, row in last_slots(batch):
        cache_np[page, row, :] = canary
    if batch.cache_dtype == "bf16":
        cache = bf16_to_device(cache_np, dev)
    else:
        cache = torch.from_numpy(cache_np).to(dev)
    qn = bf16_to_device(batch.q_nope, dev)
    qr = bf16_to_device(batch.q_rope, dev)
    idx = torch.from_numpy(np.ascontiguousarray(batch.kv_indices, dtype=np.int32)).to(dev)
    dec = PagedMlaDecoder(batch.num_heads, batch.page_size, max_batch=batch.batch,
                          kv_dtype=batch.cache_dtype, out_dtype=out_dtype, num_cus=num_cus, device=dev)
    dec.plan(batch.kv_indptr, batch.kv_last_page_len)
    scale = batch.kv_scale if kv_scale is None else kv_scale
    out, lse = dec.run_append(qn, qr, cache, idx, bf16_to_device(c_new, dev),
                              bf16_to_device(k_pe_new, dev), batch.sm_scale, scale)
    torch.cuda.synchronize()
    after = cache.cpu()
    after = after.view(torch.int16).numpy().view(np.uint16) if batch.cache_dtype == "bf16" else after.numpy()
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            after, dec)


LENS = [1, 31, 32, 33, 300, 2000]


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("ps", [1, 32, 64])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_append_parity(dev, H, ps, kv):
    batch = workloads.random_decode_batch(500 + H + ps, LENS, num_heads=H, page_size=ps, cache_dtype=kv)
    c, r = new_rows(600 + H + ps, batch.batch)
    say(f"append H={H} ps={ps} kv={kv}")
    ref_out, ref_lse, ref_cache = oracle.append_then_decode(
        batch.q_nope, batch.q_rope, batch.cache, batch.kv_indptr, batch.kv_indices,
        batch.kv_last_page_len, batch.page_size, batch.sm_scale, c, r, batch.kv_scale)
    out, lse, cache, dec = run_append(batch, dev, c, r)
    assert dec.header().num_merges > 0  # the long request is split: its last piece appends
    assert np.array_equal(cache, ref_cache), \
        f"{int((cache != ref_cache).sum())} cache elements differ from write-then-decode"
    compare(out, lse, ref_out, ref_lse, False, f"append H={H} ps={ps} kv={kv}")


@pytest.mark.parametrize("H", [16, 128])
def test_append_fp32_output(dev, H):
    batch = workloads.random_decode_batch(700 + H, [1, 64, 65, 900], num_heads=H, page_size=16)
    c, r = new_rows(701 + H, batch.batch)
    say(f"append fp32 H={H}")
    ref_out, ref_lse, ref_cache = oracle.append_then_decode(
        batch.q_nope, batch.q_rope, batch.cache, batch.kv_indptr, batch.kv_indices,
        batch.kv_last_page_len, batch.page_size, batch.sm_scale, c, r)
    out, lse, cache, _ = run_append(batch, dev, c, r, out_dtype="fp32", num_cus=4)
    assert np.array_equal(cache, ref_cache)
    compare(out, lse, ref_out, ref_lse, True, f"append fp32 H={H}")


def test_append_fp8_encoding_of_every_bf16_value(dev):
    """The device's e4m3fn encoding against the oracle's nearest-code search
    for every bf16 value of magnitude <= 448 (ties between codes, subnormals,
    zeros of both signs) and for values beyond it (clamped to +-448), with
    kv_scale 1 so that the division is exact."""
    pos = np.arange(0, 0x43E1, dtype=np.uint16)  # +0 .. 448
    big = workloads.f32_to_bf16_bits(np.array([449.0, 464.0, 480.0, 1e4, 3e38], np.float32))
    vals = np.concatenate([pos, big, pos | 0x8000, big | 0x8000])
    rows = (len(vals) + 575) // 576
    padded = np.zeros(rows * 576, dtype=np.uint16)
    padded[:len(vals)] = vals
    padded = padded.reshape(rows, 576)
    batch = workloads.random_decode_batch(800, [1] * rows, num_heads=16, page_size=1,
                                          cache_dtype="fp8_e4m3fn")
    say(f"fp8 encoding sweep: {len(vals)} values in {rows} rows")
    c, r = np.ascontiguousarray(padded[:, :512]), np.ascontiguousarray(padded[:, 512:])
    _, _, cache, _ = run_append(batch, dev, c, r, kv_scale=1.0)
    x = np.clip(workloads.bf16_bits_to_f32(padded), -448.0, 448.0)
    expect = oracle.e4m3fn_encode(x)
    for b, (page, row) in enumerate(last_slots(batch)):
        got = cache[page, row]
        bad = np.nonzero(got != expect[b])[0]
        assert bad.size == 0, (b, [(hex(padded[b, i]), hex(got[i]), hex(expect[b, i])) for i in bad[:5]])


def test_append_then_plain_decode_agree(dev):
    """After an append, a plain mla_decode over the same plan reads the stored
    rows: it must give the append call's own outputs, bit for bit."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    batch = workloads.random_decode_batch(900, [7, 128, 1000], num_heads=128, page_size=64)
    c, r = new_rows(901, batch.batch)
    say("append then plain decode")
    cache = bf16_to_device(batch.cache, dev)
    qn, qr = bf16_to_device(batch.q_nope, dev), bf16_to_device(batch.q_rope, dev)
    idx = torch.from_numpy(np.ascontiguousarray(batch.kv_indices, dtype=np.int32)).to(dev)
    dec = PagedMlaDecoder(128, 64, max_batch=batch.batch, num_cus=8, device=dev)
    dec.plan(batch.kv_indptr, batch.kv_last_page_len)
    out1, lse1 = dec.run_append(qn, qr, cache, idx, bf16_to_device(c, dev), bf16_to_device(r, dev),
                                batch.sm_scale)
    out2, lse2 = dec.run(qn, qr, cache, idx, batch.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
