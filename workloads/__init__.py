"""Seeded synthetic inputs for absorbed-MLA paged decode.

This module only draws and lays out inputs. It holds none of the method's
arithmetic: no scores, no softmax, no merge, no compaction. Both the CPU oracle
and the HIP path read what it produces. Nothing here imports either of them.

Shapes follow the workloads the pages describe:

* "MLA" on the SGLang attention-backends page: one 576-wide vector per token
  (512 latent + 64 rope) shared by all heads.
* "Paged, ragged batches" on the same page: the CSR arrays ``kv_indptr`` and
  ``kv_indices``, plus ``kv_last_page_len`` for pages larger than one token.
* Section 1 of the SGLang PR 49477 analysis: the tree mask, ``req_to_token``
  and a draft tree that is wide but shallow.

The recipe is fixed so that every run draws the same bytes:

* A numpy PCG64 generator, seeded per configuration.
* Draw order: lengths, then placement, then the absorbed query, then the rope
  query, then the cache.
* Values are N(0,1)*0.5, drawn as float32 and rounded to bfloat16 (RNE).
* Pool rows that no request references, and the tails of partially filled last
  pages, hold NaN canaries. A kernel that reads one of them poisons its output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

KV_LORA_RANK = 512
ROPE_DIM = 64
ROW = KV_LORA_RANK + ROPE_DIM  # 576 values per cached token
# DeepSeek q head = 128 nope + 64 rope, so the softmax scale is 1/sqrt(192).
SM_SCALE = 1.0 / math.sqrt(128 + 64)

BF16_NAN = np.uint16(0x7FC0)
E4M3FN_NAN = np.uint8(0x7F)
E4M3FN_MAX = 448.0

_DRAW_BLOCK_ROWS = 65536


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns. Inputs are finite by construction.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class DecodeBatch:
    """One attention-layer call of absorbed-MLA decode over a paged cache.

    Query rows ``qo_indptr[b]..qo_indptr[b+1]`` belong to request ``b`` and all
    attend to the same token list: pages ``kv_indices[kv_indptr[b]:kv_indptr[b+1]]``,
    with ``kv_last_page_len[b]`` valid tokens in the last page.
    """

    name: str
    num_heads: int
    page_size: int
    qo_indptr: np.ndarray  # int32 [B+1]
    kv_indptr: np.ndarray  # int32 [B+1]
    kv_indices: np.ndarray  # int32 [nnz_pages]
    kv_last_page_len: np.ndarray  # int32 [B]
    seq_lens: np.ndarray  # int32 [B], tokens per request (drawn lengths)
    q_nope: np.ndarray  # uint16 bf16 bits [N, H, 512] (absorbed query)
    q_rope: np.ndarray  # uint16 bf16 bits [N, H, 64]
    cache: np.ndarray  # uint16 bf16 bits or uint8 e4m3fn bytes [num_pages, page_size, 576]
    cache_dtype: str = "bf16"  # "bf16" | "fp8_e4m3fn"
    kv_scale: float = 1.0  # per-tensor dequant scale for fp8 caches
    sm_scale: float = SM_SCALE
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.kv_indptr.shape[0] - 1)

    @property
    def num_rows(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def row_seq_lens(self) -> np.ndarray:
        """Tokens attended by each query row (int64 [N])."""
        reps = np.diff(self.qo_indptr).astype(np.int64)
        return np.repeat(self.seq_lens.astype(np.int64), reps)

    @property
    def cache_bytes_per_token(self) -> int:
        return ROW * (2 if self.cache_dtype == "bf16" else 1)

    def subset(self, requests) -> "DecodeBatch":
        """The same data restricted to some requests (shares the cache pool)."""
        requests = np.asarray(requests, dtype=np.int64)
        qo = [0]
        kv = [0]
        idx = []
        qn = []
        qr = []
        for b in requests:
            q0, q1 = int(self.qo_indptr[b]), int(self.qo_indptr[b + 1])
            p0, p1 = int(self.kv_indptr[b]), int(self.kv_indptr[b + 1])
            qo.append(qo[-1] + (q1 - q0))
            kv.append(kv[-1] + (p1 - p0))
            idx.append(self.kv_indices[p0:p1])
            qn.append(self.q_nope[q0:q1])
            qr.append(self.q_rope[q0:q1])
        return dataclasses.replace(
            self,
            name=f"{self.name}[subset {len(requests)}]",
            qo_indptr=np.asarray(qo, dtype=np.int32),
            kv_indptr=np.asarray(kv, dtype=np.int32),
            kv_indices=np.concatenate(idx).astype(np.int32) if idx else np.zeros(0, np.int32),
            kv_last_page_len=self.kv_last_page_len[requests].astype(np.int32),
            seq_lens=self.seq_lens[requests].astype(np.int32),
            q_nope=np.ascontiguousarray(np.concatenate(qn)) if qn else self.q_nope[:0],
            q_rope=np.ascontiguousarray(np.concatenate(qr)) if qr else self.q_rope[:0],
        )


def _draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(0.5))


def layout_from_lengths(seq_lens: np.ndarray, page_size: int, pool_pages: int,
                        rng: np.random.Generator):
    """CSR page tables for the given lengths, pages scattered over a pool.

    The pages used are the first ``sum(ceil(L/ps))`` entries of a seeded
    permutation of the pool, handed out in request order.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    npages = (seq_lens + page_size - 1) // page_size
    need = int(npages.sum())
    if need > pool_pages:
        raise ValueError(f"pool of {pool_pages} pages cannot hold {need}")
    perm = rng.permutation(pool_pages).astype(np.int32)
    kv_indptr = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(npages)
    kv_indices = perm[:need].copy()
    last = np.where(seq_lens > 0, seq_lens - page_size * np.maximum(npages - 1, 0), 0)
    # An empty request has no pages; its last_page_len is 0 by convention.
    return kv_indptr, kv_indices, last.astype(np.int32)


def token_rows(kv_indptr, kv_indices, seq_lens, page_size) -> np.ndarray:
    """Pool row of every token, request-major (int64 [sum L])."""
    out = []
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        t = np.arange(L, dtype=np.int64)
        pages = kv_indices[int(kv_indptr[b]) + t // page_size].astype(np.int64)
        out.append(pages * page_size + t % page_size)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def fill_cache_bf16(rng, pool_pages, page_size, rows: np.ndarray) -> np.ndarray:
    """A pool of NaN canaries with fresh N(0,1)*0.5 bf16 values at ``rows``."""
    cache = np.full((pool_pages * page_size, ROW), BF16_NAN, dtype=np.uint16)
    for s in range(0, len(rows), _DRAW_BLOCK_ROWS):
        blk = rows[s:s + _DRAW_BLOCK_ROWS]
        cache[blk] = _draw_bf16(rng, (len(blk), ROW))
    return cache.reshape(pool_pages, page_size, ROW)


def quantize_e4m3fn(cache_bf16: np.ndarray, rows: np.ndarray):
    """Per-tensor fp8 e4m3fn quantisation of the used rows of a bf16 pool.

    scale = amax / 448 over the used values; code = RNE(clamp(x / scale, +-448)).
    Unused rows keep the e4m3fn NaN code as a canary. Returns (bytes, scale).
    """
    import torch

    flat = cache_bf16.reshape(-1, ROW)
    vals = bf16_bits_to_f32(flat[rows])
    amax = float(np.abs(vals).max()) if vals.size else 1.0
    scale = np.float32(amax / E4M3FN_MAX) if amax > 0 else np.float32(1.0)
    t = torch.from_numpy(vals / scale).clamp_(-E4M3FN_MAX, E4M3FN_MAX)
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    out = np.full(flat.shape, E4M3FN_NAN, dtype=np.uint8)
    out[rows] = codes
    return out.reshape(cache_bf16.shape), float(scale)


def make_decode_batch(name, seed, seq_lens_fn, num_heads, page_size, pool_pages_fn,
                      cache_dtype="bf16", rows_per_request=1, layout_only=False) -> DecodeBatch:
    """layout_only: draw the lengths and the page layout only (the same arrays
    as the full batch, since they come first in the draw order); the queries
    and the cache are then empty arrays ([N, H, 0] and [pool_pages, ps, 0])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens_fn(rng), dtype=np.int64)
    npages = (seq_lens + page_size - 1) // page_size
    pool_pages = int(pool_pages_fn(int(npages.sum())))
    kv_indptr, kv_indices, last = layout_from_lengths(seq_lens, page_size, pool_pages, rng)
    B = len(seq_lens)
    # Query rows per request: one count for all, or one per request.
    rpr = np.broadcast_to(np.asarray(rows_per_request, dtype=np.int64), (B,))
    qo_indptr = np.concatenate([[0], np.cumsum(rpr)]).astype(np.int32)
    N = int(qo_indptr[-1])
    if layout_only:
        return DecodeBatch(
            name=name, num_heads=num_heads, page_size=page_size,
            qo_indptr=qo_indptr,
            kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
            seq_lens=seq_lens.astype(np.int32), q_nope=np.zeros((N, num_heads, 0), np.uint16),
            q_rope=np.zeros((N, num_heads, 0), np.uint16),
            cache=np.zeros((pool_pages, page_size, 0), np.uint16 if cache_dtype == "bf16" else np.uint8),
            cache_dtype=cache_dtype, seed=seed)
    q_nope = _draw_bf16(rng, (N, num_heads, KV_LORA_RANK))
    q_rope = _draw_bf16(rng, (N, num_heads, ROPE_DIM))
    rows = token_rows(kv_indptr, kv_indices, seq_lens, page_size)
    cache = fill_cache_bf16(rng, pool_pages, page_size, rows)
    kv_scale = 1.0
    if cache_dtype == "fp8_e4m3fn":
        cache, kv_scale = quantize_e4m3fn(cache, rows)
    elif cache_dtype != "bf16":
        raise ValueError(cache_dtype)
    return DecodeBatch(
        name=name, num_heads=num_heads, page_size=page_size,
        qo_indptr=qo_indptr,
        kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
        seq_lens=seq_lens.astype(np.int32), q_nope=q_nope, q_rope=q_rope, cache=cache,
        cache_dtype=cache_dtype, kv_scale=kv_scale, seed=seed)


# ---------------------------------------------------------------------------
# The five workloads. Each returns a fresh, fully seeded batch.
# ---------------------------------------------------------------------------

def tiny(seed: int = 1, layout_only: bool = False) -> DecodeBatch:
    """B=2 with 7 and 33 tokens, H=16, page size 1, a pool of 64 slots."""
    return make_decode_batch(
        "tiny", seed, lambda rng: np.array([7, 33]), num_heads=16, page_size=1,
        pool_pages_fn=lambda need: 64, layout_only=layout_only)


def v2_lite(seed: int = 2, batch: int = 64, layout_only: bool = False, rows_per_request: int = 1) -> DecodeBatch:
    """DeepSeek-V2-Lite-shaped decode: H=16, page size 1, L ~ U{512..4096},
    slots scattered over a pool of 300,000. rows_per_request > 1: that many
    query rows per request over the same tokens (multi-token prediction or
    speculative decoding), drawn after the layout and before the cache."""
    name = "v2_lite" if rows_per_request == 1 else f"v2_lite_rows{rows_per_request}"
    return make_decode_batch(
        name, seed, lambda rng: rng.integers(512, 4096, size=batch, endpoint=True),
        num_heads=16, page_size=1, pool_pages_fn=lambda need: max(300_000, need),
        layout_only=layout_only, rows_per_request=rows_per_request)


def lognormal_lengths(rng, batch, median=2048.0, sigma=0.8, lo=16, hi=16384):
    z = rng.standard_normal(size=batch)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)


def v3(seed: int = 3, batch: int = 128, layout_only: bool = False) -> DecodeBatch:
    """DeepSeek-V3-shaped decode: H=128, page size 64, lognormal lengths
    (median 2048, sigma 0.8, clipped to [16, 16384]), pages permuted."""
    return make_decode_batch(
        "v3", seed, lambda rng: lognormal_lengths(rng, batch), num_heads=128, page_size=64,
        pool_pages_fn=lambda need: max(8192, need), layout_only=layout_only)


def skewed_fp8(seed: int = 5, short_len: int = 1024, long_len: int = 131072,
               batch: int = 32, layout_only: bool = False) -> DecodeBatch:
    """One very long request among short ones, H=128, page size 64, fp8 cache."""
    def lens(rng):
        L = np.full(batch, short_len, dtype=np.int64)
        L[int(rng.integers(0, batch))] = long_len
        return L
    return make_decode_batch(
        "skewed_fp8", seed, lens, num_heads=128, page_size=64,
        pool_pages_fn=lambda need: 2 * need, cache_dtype="fp8_e4m3fn", layout_only=layout_only)


@dataclasses.dataclass
class TreeVerifyBatch:
    """Tree-verify cascade inputs (PR 49477 analysis, sections 1-3).

    ``prefix`` holds every draft token as a query row (W rows per request) over
    the request's shared prefix. The draft tokens' own cache rows sit at
    ``req_to_token[r, prefix_lens[r] + j]``. ``tree_mask[r*W + i, j]`` is 1 when
    draft j is on the ancestor chain of draft i (itself included).
    """

    prefix: DecodeBatch
    width: int
    max_tree_depth: int
    parents: np.ndarray  # int32 [B, W], -1 for the root
    depth: np.ndarray  # int32 [B, W], root at depth 1
    tree_mask: np.ndarray  # uint8 [B*W, W]
    req_to_token: np.ndarray  # int32 [B, prefix + W]
    prefix_lens: np.ndarray  # int32 [B]


def random_tree(rng, width, max_depth):
    """Node 0 is the root (depth 1). Node i picks its parent uniformly among
    earlier nodes of depth < max_depth, so parents precede children."""
    parent = np.full(width, -1, dtype=np.int32)
    depth = np.zeros(width, dtype=np.int32)
    depth[0] = 1
    for i in range(1, width):
        cands = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cands[int(rng.integers(0, len(cands)))])
        parent[i] = p
        depth[i] = depth[p] + 1
    mask = np.zeros((width, width), dtype=np.uint8)
    for i in range(width):
        j = i
        while j >= 0:
            mask[i, j] = 1
            j = int(parent[j])
    return parent, depth, mask


def tree_verify(seed: int = 4, batch: int = 16, prefix_len: int = 2048, width: int = 64,
                max_depth: int = 8, num_heads: int = 128, pool_slots: int = 65536) -> TreeVerifyBatch:
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix_lens = np.full(batch, prefix_len, dtype=np.int32)
    trees = [random_tree(rng, width, max_depth) for _ in range(batch)]
    per_req = prefix_len + width
    perm = rng.permutation(pool_slots).astype(np.int32)
    req_to_token = perm[:batch * per_req].reshape(batch, per_req).copy()
    N = batch * width
    q_nope = _draw_bf16(rng, (N, num_heads, KV_LORA_RANK))
    q_rope = _draw_bf16(rng, (N, num_heads, ROPE_DIM))
    used = req_to_token.reshape(-1).astype(np.int64)
    cache = fill_cache_bf16(rng, pool_slots, 1, used)
    kv_indptr = (np.arange(batch + 1, dtype=np.int32) * prefix_len)
    kv_indices = np.ascontiguousarray(req_to_token[:, :prefix_len]).reshape(-1)
    prefix = DecodeBatch(
        name="tree_verify_prefix", num_heads=num_heads, page_size=1,
        qo_indptr=np.arange(batch + 1, dtype=np.int32) * width,
        kv_indptr=kv_indptr, kv_indices=kv_indices,
        kv_last_page_len=np.ones(batch, dtype=np.int32), seq_lens=prefix_lens.copy(),
        q_nope=q_nope, q_rope=q_rope, cache=cache, seed=seed)
    return TreeVerifyBatch(
        prefix=prefix, width=width, max_tree_depth=max_depth,
        parents=np.stack([t[0] for t in trees]), depth=np.stack([t[1] for t in trees]),
        tree_mask=np.concatenate([t[2] for t in trees]), req_to_token=req_to_token,
        prefix_lens=prefix_lens)


def random_decode_batch(seed: int, seq_lens, num_heads: int, page_size: int,
                        pool_pages: Optional[int] = None, cache_dtype: str = "bf16",
                        rows_per_request=1, layout_only: bool = False) -> DecodeBatch:
    """A small batch with explicit lengths, for parity and edge cases.
    rows_per_request: query rows of every request, or a list with one count per
    request (0 allowed). layout_only: the lengths and page layout only."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    return make_decode_batch(
        f"random(seed={seed})", seed, lambda rng: seq_lens, num_heads=num_heads,
        page_size=page_size,
        pool_pages_fn=lambda need: pool_pages if pool_pages is not None else 2 * need + 3,
        cache_dtype=cache_dtype, rows_per_request=rows_per_request, layout_only=layout_only)


@dataclasses.dataclass
class ProjectionInputs:
    """Inputs of the two per-head projections of weight absorption, bf16 bits.

    q     [N, H, D]  the no-rope query of each head, before absorption
    w_uk  [A, H, D]  latent -> key-nope map (element (a, h, d))
    w_uv  [A, H, D]  latent -> value map
    x     [N, H, A]  a latent attention output, as decode writes it
    """
    q: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    x: np.ndarray


def projection_inputs(seed: int, num_rows: int, num_heads: int,
                      head_dim: int = 128) -> ProjectionInputs:
    """Seeded projection inputs. Draw order q, w_uk, w_uv, x. Activations are
    N(0,1)*0.5 like every other input here; the weights map the 512-wide latent
    out, so they are N(0,1)/sqrt(512) (unit-variance outputs for unit inputs).
    All rounded to bfloat16 (RNE)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    A = KV_LORA_RANK
    w_scale = np.float32(1.0 / math.sqrt(A))

    def weights():
        return f32_to_bf16_bits(
            rng.standard_normal(size=(A, num_heads, head_dim), dtype=np.float32) * w_scale)

    q = _draw_bf16(rng, (num_rows, num_heads, head_dim))
    w_uk = weights()
    w_uv = weights()
    x = _draw_bf16(rng, (num_rows, num_heads, A))
    return ProjectionInputs(q=q, w_uk=w_uk, w_uv=w_uv, x=x)


CONFIGS = {
    "tiny": tiny,
    "v2_lite": v2_lite,
    "v3": v3,
    "tree_verify": tree_verify,
    "skewed_fp8": skewed_fp8,
}
