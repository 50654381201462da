"""CPU oracle for absorbed-MLA paged decode, the LSE merge and the tree-suffix compaction.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library and its
Python binding never import it, and it imports neither of them.

* ``mla_decode``: plain fp64 attention (``mla_oracle.c``), built with gcc.
* ``merge_states``: the two-state log-sum-exp merge (``mla_oracle.c``).
* ``absorb_query`` / ``project_output``: the per-head W_UK and W_UV products on
  either side of the latent attention (numpy matrix products in float64).
* ``e4m3fn_encode`` / ``append_then_decode``: the fused KV-cache update, written
  as what it must equal: store the new token's row (bf16, or e4m3fn codes
  chosen as the nearest code to value / scale), then decode.
* ``quantize_query_e4m3fn``: the query of the optional fp8 score, as its
  definition: per (row, head) a power-of-two scale and the nearest e4m3fn code
  of every scaled value. The decode with that score is ``mla_decode`` on the
  dequantized query, since the query enters only the score.
* ``tree_suffix_compact``: the pre-PR definition of the suffix page table from
  section 1 of the SGLang PR 49477 analysis: sort the keys "column if visible,
  column + W if not" with a stable sort, gather the draft slots in that order,
  and count the visible ones.

Every function is pinned by tests under ``tests/`` against things other than
itself: the absorption identity, a library attention routine, closed forms,
brute force and the pages' own arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")
_lock = threading.Lock()
_lib = None

CACHE_BF16, CACHE_F64, CACHE_E4M3FN = 0, 1, 2
LATENT, ROPE = 512, 64


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (no fast-math, OpenMP). Returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            p = ctypes.c_void_p
            i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
            lib.oracle_mla_decode.restype = i32
            lib.oracle_mla_decode.argtypes = [i32, i32, i32, p, p, p, p, p, p, p, i32, f64, f64, p, p]
            lib.oracle_merge_states.restype = None
            lib.oracle_merge_states.argtypes = [i64, i32, p, p, p, p, p, p]
            lib.oracle_decode_elements.restype = None
            lib.oracle_decode_elements.argtypes = [i32, p, i64, p]
            lib.oracle_num_threads.restype = i32
            lib.oracle_num_threads.argtypes = []
            lib.oracle_set_num_threads.restype = None
            lib.oracle_set_num_threads.argtypes = [i32]
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the next oracle calls; n <= 0 restores the default (all cores)."""
    _load().oracle_set_num_threads(int(n))


def bf16_to_double(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_decode_elements(CACHE_BF16, _ptr(bits), bits.size, _ptr(out))
    return out


def e4m3fn_to_double(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_decode_elements(CACHE_E4M3FN, _ptr(codes), codes.size, _ptr(out))
    return out


def mla_decode(q_nope, q_rope, cache, kv_indptr, kv_indices, page_size, sm_scale,
               kv_last_page_len=None, qo_indptr=None, kv_scale=1.0):
    """Absorbed-MLA decode in fp64. Returns (out [N,H,512], lse [N,H]) as float64.

    ``q_nope``/``q_rope`` are float64 arrays, or uint16 bfloat16 bit patterns
    (widened exactly). ``cache`` is [pages, page_size, 576] of uint16 bf16
    bits, uint8 e4m3fn codes (times ``kv_scale``) or float64.
    """
    q_nope = np.asarray(q_nope)
    q_rope = np.asarray(q_rope)
    if q_nope.dtype == np.uint16:
        q_nope = bf16_to_double(q_nope)
    if q_rope.dtype == np.uint16:
        q_rope = bf16_to_double(q_rope)
    q_nope = np.ascontiguousarray(q_nope, dtype=np.float64)
    q_rope = np.ascontiguousarray(q_rope, dtype=np.float64)
    N, H, A = q_nope.shape
    assert A == LATENT and q_rope.shape == (N, H, ROPE), (q_nope.shape, q_rope.shape)
    cache = np.ascontiguousarray(cache)
    assert cache.shape[-1] == LATENT + ROPE
    dtype = {np.dtype(np.uint16): CACHE_BF16, np.dtype(np.uint8): CACHE_E4M3FN,
             np.dtype(np.float64): CACHE_F64}[cache.dtype]
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    B = kv_indptr.shape[0] - 1
    if qo_indptr is not None:
        qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int32)
        assert qo_indptr[-1] == N
    else:
        assert N == B
    if kv_last_page_len is not None:
        kv_last_page_len = np.ascontiguousarray(kv_last_page_len, dtype=np.int32)
    out = np.empty((N, H, LATENT), dtype=np.float64)
    lse = np.empty((N, H), dtype=np.float64)
    rc = _load().oracle_mla_decode(
        B, H, int(page_size), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
        _ptr(kv_last_page_len), _ptr(q_nope), _ptr(q_rope), _ptr(cache), dtype,
        float(kv_scale), float(sm_scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_mla_decode rejected the layout")
    return out, lse


def decode_batch(batch):
    """``mla_decode`` on a ``workloads.DecodeBatch``-shaped object."""
    return mla_decode(batch.q_nope, batch.q_rope, batch.cache, batch.kv_indptr, batch.kv_indices,
                      batch.page_size, batch.sm_scale, kv_last_page_len=batch.kv_last_page_len,
                      qo_indptr=batch.qo_indptr, kv_scale=batch.kv_scale)


def e4m3fn_encode(x) -> np.ndarray:
    """Nearest OCP e4m3fn code to each value, ties to the code with an even
    mantissa (round to nearest even), by direct search over the decoded values
    of the 127 non-negative finite codes. Values must be finite with
    |x| <= 448; the sign bit of x (including -0.0) becomes the code's sign."""
    x = np.asarray(x, dtype=np.float64)
    assert np.isfinite(x).all() and (np.abs(x) <= 448.0).all()
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E, ascending in value
    vals = e4m3fn_to_double(codes)
    a = np.abs(x).ravel()
    hi = np.minimum(np.searchsorted(vals, a, side="left"), 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = (d_hi == d_lo) & (hi != lo)
    pick = np.where(tie, np.where(hi % 2 == 0, hi, lo), pick)
    pick = np.where(a == vals[hi], hi, pick)
    sign = np.signbit(x).ravel().astype(np.uint8) << 7
    return (pick.astype(np.uint8) | sign).reshape(x.shape)


def quantize_query_e4m3fn(q_nope, q_rope):
    """Query of the optional fp8 score (an fp8 matrix-core product of the
    query with an e4m3fn cache; the pages leave the query's quantisation open).

    Per query row n and head h, over the head's 576 values (the 512 absorbed
    no-rope values, then the 64 rope values): amax is the largest magnitude
    and e the smallest integer with amax * 2^-e <= 448 (e = 0 for a head of
    zeros). Every value is scaled by 2^-e, which is exact, and encoded as its
    nearest e4m3fn code (``e4m3fn_encode``). The score then multiplies the
    dequantized query q_hat = code value * 2^e.

    ``q_nope`` [N,H,512] and ``q_rope`` [N,H,64] are bf16 bit patterns (uint16)
    or float64. Returns (codes_nope uint8, codes_rope uint8, e int32 [N,H],
    q_hat_nope float64, q_hat_rope float64)."""
    qn = np.asarray(q_nope)
    qr = np.asarray(q_rope)
    qn = bf16_to_double(qn) if qn.dtype == np.uint16 else np.asarray(qn, np.float64)
    qr = bf16_to_double(qr) if qr.dtype == np.uint16 else np.asarray(qr, np.float64)
    q = np.concatenate([qn, qr], axis=-1)
    amax = np.abs(q).max(axis=-1)
    e = np.zeros(amax.shape, dtype=np.int64)
    for idx in zip(*np.nonzero(amax > 0)):
        a = float(amax[idx])
        k = int(np.floor(np.log2(a))) - 9  # a first guess; the two loops make it exact
        while np.ldexp(a, -k) > 448.0:
            k += 1
        while np.ldexp(a, -(k - 1)) <= 448.0:
            k -= 1
        e[idx] = k
    codes = e4m3fn_encode(np.ldexp(q, -e[..., None]))
    q_hat = np.ldexp(e4m3fn_to_double(codes), e[..., None])
    return (codes[..., :LATENT], codes[..., LATENT:], e.astype(np.int32),
            q_hat[..., :LATENT], q_hat[..., LATENT:])


def append_then_decode(q_nope, q_rope, cache, kv_indptr, kv_indices, kv_last_page_len, page_size,
                       sm_scale, c_new, k_pe_new, kv_scale=1.0):
    """The fused append (sglang-jax MLA gap page, section 2.4: the kernel
    updates the cache with the new token; section 3.1: latent and rope parts
    written separately) as its definition: each request b (one query row per
    request) stores its new token at position L_b - 1, where L_b counts it,
    then attends over all L_b tokens. For a bf16 cache the row is the bf16
    inputs; for an e4m3fn cache each value is v / kv_scale (a float32
    division), clamped to +-448 and encoded by ``e4m3fn_encode``.

    ``c_new`` [B, 512] and ``k_pe_new`` [B, 64] are bf16 bit patterns. Returns
    (out, lse, cache_after) with cache_after a new array."""
    cache = np.array(cache, copy=True)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    B = len(kv_indptr) - 1
    npages = kv_indptr[1:] - kv_indptr[:-1]
    lens = np.where(npages > 0, (npages - 1) * page_size + last, 0)
    assert (lens >= 1).all(), "every request holds its new token"
    row_bits = np.concatenate([np.asarray(c_new, np.uint16), np.asarray(k_pe_new, np.uint16)], axis=1)
    for b in range(B):
        tok = int(lens[b]) - 1
        page = int(kv_indices[kv_indptr[b] + tok // page_size])
        if cache.dtype == np.uint16:
            cache[page, tok % page_size, :] = row_bits[b]
        else:
            v = bf16_to_double(row_bits[b]).astype(np.float32) / np.float32(kv_scale)
            cache[page, tok % page_size, :] = e4m3fn_encode(np.clip(v, -448.0, 448.0))
    out, lse = mla_decode(q_nope, q_rope, cache, kv_indptr, kv_indices, page_size, sm_scale,
                          kv_last_page_len=last, kv_scale=kv_scale)
    return out, lse, cache


def absorb_query(q_nope, w_uk):
    """W_UK absorption into the query (SGLang v0.3 MLA page, weight absorption;
    sglang-jax MLA gap page, section 2.1): per head, the 128-wide nope query
    times W_UK^T gives the 512-wide query that scores directly against the
    latent. q_nope [N, H, D], w_uk [A, H, D] (the [A, N, H] layout of the gap
    page's MLAEinsum split, section 2.2) -> q_abs [N, H, A] float64.
    q_abs[n, h, a] = sum_d q_nope[n, h, d] * w_uk[a, h, d]."""
    q = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    N, H, D = q.shape
    A = w.shape[0]
    assert w.shape == (A, H, D)
    out = np.empty((N, H, A))
    for h in range(H):  # one matrix product per head
        out[:, h, :] = q[:, h, :] @ w[:, h, :].T
    return out


def project_output(out_latent, w_uv):
    """W_UV applied after the latent attention (the same pages: W_UV moves to the
    output side): per head, the 512-wide latent output times W_UV gives the
    head_dim-wide value output. out_latent [N, H, A], w_uv [A, H, D] ->
    o [N, H, D] float64. o[n, h, d] = sum_a out_latent[n, h, a] * w_uv[a, h, d]."""
    x = np.asarray(out_latent, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    N, H, A = x.shape
    D = w.shape[2]
    assert w.shape == (A, H, D)
    o = np.empty((N, H, D))
    for h in range(H):
        o[:, h, :] = x[:, h, :] @ w[:, h, :]
    return o


def merge_states(v_a, s_a, v_b, s_b):
    """LSE merge of two states. v: [..., d] float64, s: [...] float64."""
    v_a = np.ascontiguousarray(v_a, dtype=np.float64)
    v_b = np.ascontiguousarray(v_b, dtype=np.float64)
    s_a = np.ascontiguousarray(s_a, dtype=np.float64)
    s_b = np.ascontiguousarray(s_b, dtype=np.float64)
    assert v_a.shape == v_b.shape and s_a.shape == s_b.shape == v_a.shape[:-1]
    d = v_a.shape[-1]
    n = int(np.prod(s_a.shape)) if s_a.ndim else 1
    v = np.empty_like(v_a)
    s = np.empty_like(s_a)
    _load().oracle_merge_states(n, d, _ptr(v_a), _ptr(s_a), _ptr(v_b), _ptr(s_b), _ptr(v), _ptr(s))
    return v, s


def tree_suffix_compact(tree_mask, req_to_token, prefix_lens, width, rows=None,
                        num_actual_rows=None):
    """Suffix page table and sequence lengths for tree-verify attention.

    Query row ``r`` belongs to request ``r // width``. Its draft slots are
    ``req_to_token[req, prefix_lens[req] + j]`` for j < width. Following the
    pre-PR definition: keys = where(mask, col, col + width); order = stable
    argsort(keys); table[r] = slots[order]; seqlens[r] = mask[r].sum().
    Rows at or past ``num_actual_rows`` (graph padding) read no mask and get a
    zero table row and length 0.
    """
    tree_mask = np.asarray(tree_mask).astype(bool)
    req_to_token = np.asarray(req_to_token, dtype=np.int32)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    n_actual = tree_mask.shape[0] if num_actual_rows is None else int(num_actual_rows)
    rows = n_actual if rows is None else int(rows)
    table = np.zeros((rows, width), dtype=np.int32)
    seqlens = np.zeros(rows, dtype=np.int32)
    cols = np.arange(width)
    for r in range(min(rows, n_actual)):
        req = r // width
        m = tree_mask[r, :width]
        keys = np.where(m, cols, cols + width)
        order = np.argsort(keys, kind="stable")
        slots = req_to_token[req, prefix_lens[req] + cols]
        table[r] = slots[order]
        seqlens[r] = int(m.sum())
    return table, seqlens
