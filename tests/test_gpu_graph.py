"""Graph-safe decode (MLA_DECODE_GRAPH_SAFE): one call captured in a HIP graph,
replayed after each new plan is built into the same workspace, must give what
an eager call on that plan gives, bit for bit, and what the oracle gives
within the tolerances. Between replays the test does eager work of its own and
synchronises, and every replay is checked. Plans with fewer query rows leave
the output rows past them untouched (padding)."""
import dataclasses

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


@pytest.mark.parametrize("H,fp8_score", [(16, False), (128, False), (128, True)])
def test_graph_replay_follows_the_plan(dev, H, fp8_score):
    """fp8_score: an e4m3fn pool and MLA_DECODE_FP8_SCORE, whose query
    quantisation launch is captured with the decode and merges."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    ps, B = 16, 6
    # One pool holds every batch's tokens: batch k uses its own page list of it.
    lens_set = [[3000, 40, 1, 700, 64, 2000], [10, 5000, 300, 0, 33, 17], [900, 900, 1]]
    kv = "fp8_e4m3fn" if fp8_score else "bf16"
    pool = workloads.random_decode_batch(90 + H, [12000], num_heads=H, page_size=ps, cache_dtype=kv)
    cache = torch.from_numpy(pool.cache).to(dev) if fp8_score else bf16_to_device(pool.cache, dev)
    rng = np.random.Generator(np.random.PCG64(91))
    q_all = workloads.f32_to_bf16_bits(rng.standard_normal((B, H, 576), dtype=np.float32) * np.float32(0.5))
    q = bf16_to_device(q_all, dev)
    qn, qr = q[:, :, :512], q[:, :, 512:]
    filled = pool.kv_indices  # the pool pages that hold values (the rest are NaN canaries)

    def csr(lens, seed):
        r = np.random.Generator(np.random.PCG64(seed))
        npages = [(L + ps - 1) // ps for L in lens]
        indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
        indices = filled[r.permutation(len(filled))[:indptr[-1]]].astype(np.int32)
        last = np.array([L - ps * (n - 1) if L > 0 else 0 for L, n in zip(lens, npages)], np.int32)
        return indptr, indices, last

    batches = [csr(lens, 100 + k) for k, lens in enumerate(lens_set)]

    def oracle_batch(k):
        """Batch k over the shared pool, as a DecodeBatch for the oracle."""
        indptr, indices, last = batches[k]
        n = len(lens_set[k])
        return dataclasses.replace(
            pool, qo_indptr=np.arange(n + 1, dtype=np.int32), kv_indptr=indptr, kv_indices=indices,
            kv_last_page_len=last, seq_lens=np.asarray(lens_set[k], np.int32),
            q_nope=np.ascontiguousarray(q_all[:n, :, :512]), q_rope=np.ascontiguousarray(q_all[:n, :, 512:]))

    def check_oracle(k, o, l, what):
        b = oracle_batch(k)
        n = b.num_rows
        o = o[:n].float().cpu().numpy().astype(np.float64)
        l = l[:n].cpu().numpy().astype(np.float64)
        if fp8_score:
            from test_gpu_fp8_score import check, reference
            ref_out, ref_lse, D, M = reference(b)
            check(o, l, ref_out, ref_lse, D, M, what)
        else:
            ref_out, ref_lse = oracle.decode_batch(b)
            compare(o, l, ref_out, ref_lse, False, what)
    max_idx = max(len(b[1]) for b in batches)
    idx = torch.zeros(max_idx, dtype=torch.int32, device=dev)  # fixed buffer the graph reads
    dec = PagedMlaDecoder(H, ps, max_batch=B, num_cus=16, device=dev, graph_safe=True, kv_dtype=kv,
                          fp8_score=fp8_score)
    out = torch.zeros((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((B, H), dtype=torch.float32, device=dev)

    def load(k):
        indptr, indices, last = batches[k]
        idx[:len(indices)].copy_(torch.from_numpy(indices))
        return dec.plan(indptr, last)

    h0 = load(0)
    assert h0.num_merges > 0
    dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale, out=out, lse=lse)  # warm up outside the capture
    torch.cuda.synchronize()
    check_oracle(0, out, lse, f"H={H} fp8_score={fp8_score} graph-safe eager call vs oracle")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep, k in enumerate([1, 0, 2, 1, 2, 0]):
        h = load(k)
        rows = h.num_rows
        sentinel_out = out[rows:].clone()
        sentinel_lse = lse[rows:].clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale)  # eager, same plan
        torch.cuda.synchronize()
        say(f"H={H} fp8_score={fp8_score} replay {rep}: batch {k} rows={rows} merges={h.num_merges} wide={h.num_wide_merges}")
        assert torch.equal(out[:rows], ref_out[:rows]) and torch.equal(lse[:rows], ref_lse[:rows]), \
            f"replay {rep} (batch {k}) differs from the eager call"
        check_oracle(k, out, lse, f"replay {rep} vs oracle")
        assert torch.equal(out[rows:], sentinel_out) and torch.equal(lse[rows:], sentinel_lse), \
            "padding rows were written"
        out[:rows].zero_()  # eager work between replays


def test_tree_verify_step_replays_from_one_graph(dev):
    """Configuration 4's step (compaction, then the single pass) captured once
    and replayed for new draft trees and new prefix lengths: buffers sized for
    the largest batch, padding rows past the live ones, plans rebuilt between
    replays. Every replay must equal the eager step on the same inputs."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder, tree_suffix_compact
    B, W, D, H = 4, 64, 8, 128
    trees = [workloads.tree_verify(seed=40 + k, batch=B, prefix_len=300 + 37 * k, width=W, max_depth=D,
                                   pool_slots=8192) for k in range(3)]
    N = B * W
    rows_pad = N + 16  # graph padding rows: the compaction zeroes them, the decode never plans them
    base = trees[0].prefix
    cache = bf16_to_device(base.cache, dev)  # one pool; every tree's slots hold values in it
    pool_h = base.cache.reshape(-1, 576).copy()  # the same pool on the host, for the oracle
    for t in trees[1:]:
        used = np.unique(t.req_to_token)
        cache.view(-1, 576)[torch.from_numpy(used.astype(np.int64)).to(dev)] = \
            bf16_to_device(t.prefix.cache.reshape(-1, 576)[used], dev)
        pool_h[used] = t.prefix.cache.reshape(-1, 576)[used]
    qn = torch.zeros((rows_pad, H, 512), dtype=torch.bfloat16, device=dev)
    qr = torch.zeros((rows_pad, H, 64), dtype=torch.bfloat16, device=dev)
    mask = torch.zeros((N, W), dtype=torch.uint8, device=dev)
    r2t = torch.zeros(trees[0].req_to_token.shape[0], 2048, dtype=torch.int32, device=dev)
    plen = torch.zeros(B, dtype=torch.int32, device=dev)
    idx = torch.zeros(B * 2048, dtype=torch.int32, device=dev)
    dec = PagedMlaDecoder(H, 1, max_batch=B, max_rows=N, device=dev, graph_safe=True, suffix_tokens=D)
    out = torch.zeros((N, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((N, H), dtype=torch.float32, device=dev)

    def load(t):
        p = t.prefix
        qn[:N].copy_(bf16_to_device(p.q_nope, dev))
        qr[:N].copy_(bf16_to_device(p.q_rope, dev))
        mask.copy_(torch.from_numpy(t.tree_mask))
        r2t.zero_()
        r2t[:, :t.req_to_token.shape[1]].copy_(torch.from_numpy(t.req_to_token))
        plen.copy_(torch.from_numpy(t.prefix_lens))
        idx.zero_()
        idx[:len(p.kv_indices)].copy_(torch.from_numpy(p.kv_indices))
        dec.plan(p.kv_indptr, p.kv_last_page_len, p.qo_indptr)

    def step(o, l):
        table, seqlens = tree_suffix_compact(mask, r2t, plen, W, num_rows=rows_pad, num_actual_rows=N)
        dec.run_tree_verify(qn, qr, cache, idx, table, seqlens, base.sm_scale, out=o, lse=l)

    load(trees[0])
    step(out, lse)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        step(out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep, k in enumerate([1, 2, 0, 2]):
        load(trees[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_o = torch.empty_like(out)
        ref_l = torch.empty_like(lse)
        step(ref_o, ref_l)
        torch.cuda.synchronize()
        say(f"tree replay {rep}: tree {k}, prefix {int(trees[k].prefix_lens[0])}")
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs"
        # Every row against the oracle: its prefix, then its visible drafts.
        t = trees[k]
        p = t.prefix
        kv_indptr, kv_indices = [0], []
        for r in range(N):
            req, pl = r // W, int(t.prefix_lens[r // W])
            vis = np.nonzero(t.tree_mask[r])[0]
            kv_indices.append(np.concatenate([t.req_to_token[req, :pl], t.req_to_token[req, pl + vis]]))
            kv_indptr.append(kv_indptr[-1] + len(kv_indices[-1]))
        ref_out, ref_lse = oracle.mla_decode(
            p.q_nope, p.q_rope, pool_h.reshape(-1, 1, 576), np.asarray(kv_indptr, np.int32),
            np.concatenate(kv_indices).astype(np.int32), 1, base.sm_scale,
            kv_last_page_len=np.ones(N, np.int32))
        compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                ref_out, ref_lse, False, f"tree replay {rep} vs oracle")
        out.zero_()


@pytest.mark.parametrize("H", [16, 32])
def test_graph_replay_with_shared_rows(dev, H):
    """Graph-safe plans with MLA_DECODE_SHARED_ROWS: batches with different row
    counts per request through one captured call; each replay equals an eager
    call on its plan bit for bit and the oracle within the tolerances, and rows
    past the plan's are left as they were."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    ps = 16
    cases = [([3000, 40, 1, 700], [4, 1, 2, 3]), ([10, 5000, 300], [1, 5, 2]), ([900, 900], [2, 2])]
    max_rows = max(sum(r) for _, r in cases)
    max_batch = max(len(lens) for lens, _ in cases)
    pool = workloads.random_decode_batch(95 + H, [12000], num_heads=H, page_size=ps)
    cache = bf16_to_device(pool.cache, dev)
    rng = np.random.Generator(np.random.PCG64(96))
    q_all = workloads.f32_to_bf16_bits(rng.standard_normal((max_rows, H, 576), dtype=np.float32) * np.float32(0.5))
    q = bf16_to_device(q_all, dev)
    qn, qr = q[:, :, :512], q[:, :, 512:]
    filled = pool.kv_indices

    def csr(lens, rows, seed):
        r = np.random.Generator(np.random.PCG64(seed))
        npages = [(L + ps - 1) // ps for L in lens]
        indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
        indices = filled[r.permutation(len(filled))[:indptr[-1]]].astype(np.int32)
        last = np.array([L - ps * (n - 1) if L > 0 else 0 for L, n in zip(lens, npages)], np.int32)
        qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        return indptr, indices, last, qo

    batches = [csr(lens, rows, 200 + k) for k, (lens, rows) in enumerate(cases)]

    def check_oracle(k, o, l, what):
        indptr, indices, last, qo = batches[k]
        n = int(qo[-1])
        b = dataclasses.replace(
            pool, qo_indptr=qo, kv_indptr=indptr, kv_indices=indices, kv_last_page_len=last,
            seq_lens=np.asarray(cases[k][0], np.int32),
            q_nope=np.ascontiguousarray(q_all[:n, :, :512]), q_rope=np.ascontiguousarray(q_all[:n, :, 512:]))
        ref_out, ref_lse = oracle.decode_batch(b)
        compare(o[:n].float().cpu().numpy().astype(np.float64), l[:n].cpu().numpy().astype(np.float64),
                ref_out, ref_lse, False, what)

    max_idx = max(len(b[1]) for b in batches)
    idx = torch.zeros(max_idx, dtype=torch.int32, device=dev)
    dec = PagedMlaDecoder(H, ps, max_batch=max_batch, max_rows=max_rows, num_cus=16, device=dev,
                          graph_safe=True, shared_rows=True)
    out = torch.zeros((max_rows, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((max_rows, H), dtype=torch.float32, device=dev)

    def load(k):
        indptr, indices, last, qo = batches[k]
        idx[:len(indices)].copy_(torch.from_numpy(indices))
        return dec.plan(indptr, last, qo)

    h0 = load(0)
    assert h0.num_merges > 0
    dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    check_oracle(0, out, lse, f"H={H} shared rows graph-safe eager call vs oracle")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep, k in enumerate([1, 2, 0, 2, 1]):
        h = load(k)
        rows = h.num_rows
        sentinel_out = out[rows:].clone()
        sentinel_lse = lse[rows:].clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale)
        torch.cuda.synchronize()
        say(f"H={H} shared rows replay {rep}: batch {k} rows={rows} items={h.num_items} merges={h.num_merges}")
        assert torch.equal(out[:rows], ref_out[:rows]) and torch.equal(lse[:rows], ref_lse[:rows]), \
            f"replay {rep} (batch {k}) differs from the eager call"
        check_oracle(k, out, lse, f"replay {rep} vs oracle")
        assert torch.equal(out[rows:], sentinel_out) and torch.equal(lse[rows:], sentinel_lse), \
            "padding rows were written"
        out[:rows].zero_()


@pytest.mark.parametrize("H,shared,ps", [(16, False, 16), (32, True, 16), (128, False, 16), (128, False, 64)])
def test_graph_replay_over_random_plans(dev, H, shared, ps):
    """One captured graph-safe call replayed over eight random plans (request
    counts, lengths from empty to long, row counts, splits): each replay equal
    to an eager call bit for bit and to the oracle within the tolerances. At
    128 heads and 64 tokens per page the decode takes the page-uniform tiles."""
    from paged_mla_decode_amd.decoder import PagedMlaDecoder
    max_batch, max_rows = 8, 24
    # Whole pages only: a partly filled last page holds NaN canaries in its tail,
    # and the cases below use the pool's pages as full pages.
    pool = workloads.random_decode_batch(120 + H, [ps * -(-50000 // ps)], num_heads=H, page_size=ps)
    cache = bf16_to_device(pool.cache, dev)
    rng = np.random.Generator(np.random.PCG64(121 + H))
    q_all = workloads.f32_to_bf16_bits(rng.standard_normal((max_rows, H, 576), dtype=np.float32) * np.float32(0.5))
    q = bf16_to_device(q_all, dev)
    qn, qr = q[:, :, :512], q[:, :, 512:]
    filled = pool.kv_indices
    cases = []
    for k in range(8):
        B = int(rng.integers(1, max_batch + 1))
        lens = [int(x) for x in rng.choice([0, 1, 33, 300, 2000, 6000], size=B)]
        rows = [int(x) for x in rng.integers(1, 4, size=B)]
        while sum(rows) > max_rows:
            rows[int(np.argmax(rows))] -= 1
        npages = [(L + ps - 1) // ps for L in lens]
        indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
        assert indptr[-1] <= len(filled)  # distinct pages that hold values
        indices = filled[rng.permutation(len(filled))[:indptr[-1]]].astype(np.int32)
        last = np.array([L - ps * (n - 1) if L > 0 else 0 for L, n in zip(lens, npages)], np.int32)
        qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        cases.append((lens, indptr, indices, last, qo))
    idx = torch.zeros(max(1, max(len(c[2]) for c in cases)), dtype=torch.int32, device=dev)
    dec = PagedMlaDecoder(H, ps, max_batch=max_batch, max_rows=max_rows, num_cus=32, device=dev,
                          graph_safe=True, shared_rows=shared)
    out = torch.zeros((max_rows, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((max_rows, H), dtype=torch.float32, device=dev)

    def load(k):
        lens, indptr, indices, last, qo = cases[k]
        if len(indices):
            idx[:len(indices)].copy_(torch.from_numpy(indices))
        return dec.plan(indptr, last, qo)

    load(0)
    dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(len(cases)):
        h = load(k)
        rows = h.num_rows
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = dec.run(qn, qr, cache, idx, pool.sm_scale, pool.kv_scale)
        torch.cuda.synchronize()
        lens, indptr, indices, last, qo = cases[k]
        say(f"H={H} shared={shared} ps={ps} random plan {k}: lens={lens} rows={np.diff(qo).tolist()} "
            f"items={h.num_items} merges={h.num_merges} wide={h.num_wide_merges}")
        assert torch.equal(out[:rows], ref_out[:rows]) and torch.equal(lse[:rows], ref_lse[:rows]), \
            f"replay {k} differs from the eager call"
        b = dataclasses.replace(
            pool, qo_indptr=qo, kv_indptr=indptr, kv_indices=indices, kv_last_page_len=last,
            seq_lens=np.asarray(lens, np.int32),
            q_nope=np.ascontiguousarray(q_all[:rows, :, :512]), q_rope=np.ascontiguousarray(q_all[:rows, :, 512:]))
        o_ref, l_ref = oracle.decode_batch(b)
        compare(out[:rows].float().cpu().numpy().astype(np.float64), lse[:rows].cpu().numpy().astype(np.float64),
                o_ref, l_ref, False, f"random plan {k} replay vs oracle")
        out[:rows].zero_()
