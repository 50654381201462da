"""Convenience wrapper around the C ABI: owns the pinned host plan buffer and
the device workspace (torch allocations), and calls mla_decode_plan /
mla_decode. Every step of the computation runs in the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _binding as B

_DTYPES = {"bf16": B.MLA_DTYPE_BF16, "fp32": B.MLA_DTYPE_FP32, "fp8_e4m3fn": B.MLA_DTYPE_FP8_E4M3FN}


class PagedMlaDecoder:
    """Absorbed-MLA decode over a paged latent cache for batches of up to
    ``max_batch`` requests and ``max_rows`` query rows."""

    def __init__(self, num_heads: int, page_size: int, max_batch: int, max_rows: int | None = None,
                 kv_dtype: str = "bf16", out_dtype: str = "bf16", num_cus: int = 0,
                 max_splits: int = 0, device="cuda", graph_safe: bool = False,
                 suffix_tokens: int = 0, fp8_score: bool = False, shared_rows: bool = False):
        self.device = torch.device(device)
        max_rows = max_batch if max_rows is None else max_rows
        # Graph-safe: launches and workspace addresses fixed for up to max_rows rows.
        # fp8_score: the score on the fp8 matrix core with an e4m3fn-quantised query.
        # shared_rows: a request's query rows share each tile (16 and 32 heads).
        flags = ((B.MLA_DECODE_GRAPH_SAFE if graph_safe else 0) | (B.MLA_DECODE_FP8_SCORE if fp8_score else 0)
                 | (B.MLA_DECODE_SHARED_ROWS if shared_rows else 0))
        self.params = B.make_params(num_heads, page_size, _DTYPES[kv_dtype], _DTYPES[out_dtype],
                                    num_cus, max_splits,
                                    flags=flags,
                                    max_rows=max_rows if graph_safe else 0,
                                    suffix_tokens=suffix_tokens)
        self.kv_dtype = kv_dtype
        self.out_dtype = out_dtype
        self.num_heads = num_heads
        max_rows = max_batch if max_rows is None else max_rows
        plan_bytes, ws_bytes = B.mla_decode_workspace_size(self.params, max_batch, max_rows)
        self.plan_h = torch.empty(plan_bytes, dtype=torch.uint8, pin_memory=True)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        self._copy_done = None
        self._header = None
        self.variant = B.mla_decode_variant(self.params)

    def plan(self, kv_indptr, kv_last_page_len=None, qo_indptr=None, stream=None):
        """Build the plan for a batch (host arrays) and copy it to the workspace."""
        kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
        last = None if kv_last_page_len is None else np.ascontiguousarray(kv_last_page_len, np.int32)
        qo = None if qo_indptr is None else np.ascontiguousarray(qo_indptr, dtype=np.int32)
        if self._copy_done is not None:  # the previous plan copy still reads plan_h
            self._copy_done.synchronize()
        stream = stream or torch.cuda.current_stream(self.device)
        st = B.mla_decode_plan(self.params, len(kv_indptr) - 1, qo, kv_indptr, last, self.plan_h,
                               self.plan_h.numel(), self.workspace, self.workspace.numel(), stream)
        if st != B.MLA_OK:
            raise B.MlaError("mla_decode_plan", st)
        self._copy_done = torch.cuda.Event()
        self._copy_done.record(stream)
        self._header = B.read_plan(self.plan_h)[0]
        return self._header

    def header(self):
        return self._header

    def run(self, q_nope, q_rope, kv_cache, kv_indices, sm_scale, kv_scale=1.0, kv_lens=None,
            out=None, lse=None, stream=None):
        """out [N, H, 512] (bf16 or fp32) and lse [N, H] fp32 for the planned batch.

        q_nope/q_rope: bf16 [N, H, 512] / [N, H, 64] (any strides with a unit last
        dim). kv_cache: [pages, page_size, 576] bf16, or uint8 e4m3fn codes.
        """
        h = self.header()
        N, H = h.num_rows, self.num_heads
        if out is None:
            dt = torch.float32 if self.out_dtype == "fp32" else torch.bfloat16
            out = torch.empty((N, H, 512), dtype=dt, device=self.device)
        if lse is None:
            lse = torch.empty((N, H), dtype=torch.float32, device=self.device)
        assert q_nope.stride(-1) == 1 and q_rope.stride(-1) == 1
        stream = stream or torch.cuda.current_stream(self.device)
        st = B.mla_decode(self.params, self.plan_h, self.workspace, self.workspace.numel(), q_nope,
                          q_nope.stride(0), q_nope.stride(1), q_rope, q_rope.stride(0),
                          q_rope.stride(1), kv_cache, kv_scale, kv_indices, kv_lens, sm_scale, out,
                          lse, stream)
        if st != B.MLA_OK:
            raise B.MlaError("mla_decode", st)
        return out, lse


    def run_append(self, q_nope, q_rope, kv_cache, kv_indices, c_new, k_pe_new, sm_scale,
                   kv_scale=1.0, out=None, lse=None, stream=None):
        """``run`` with each request's new token written into its cache row L-1
        first, in the same launch (mla_decode_append). c_new [N, 512] and
        k_pe_new [N, 64] bf16, unit last stride; one query row per request."""
        h = self.header()
        N, H = h.num_rows, self.num_heads
        if out is None:
            dt = torch.float32 if self.out_dtype == "fp32" else torch.bfloat16
            out = torch.empty((N, H, 512), dtype=dt, device=self.device)
        if lse is None:
            lse = torch.empty((N, H), dtype=torch.float32, device=self.device)
        assert q_nope.stride(-1) == 1 and q_rope.stride(-1) == 1
        assert c_new.stride(-1) == 1 and k_pe_new.stride(-1) == 1
        stream = stream or torch.cuda.current_stream(self.device)
        st = B.mla_decode_append(self.params, self.plan_h, self.workspace, self.workspace.numel(),
                                 q_nope, q_nope.stride(0), q_nope.stride(1), q_rope,
                                 q_rope.stride(0), q_rope.stride(1), kv_cache, kv_scale,
                                 kv_indices, c_new, c_new.stride(0), k_pe_new, k_pe_new.stride(0),
                                 sm_scale, out, lse, stream)
        if st != B.MLA_OK:
            raise B.MlaError("mla_decode_append", st)
        return out, lse


    def run_suffix_merge(self, q_nope, q_rope, kv_cache, kv_indices, sm_scale, prefix_out,
                         prefix_lse, kv_scale=1.0, kv_lens=None, out=None, lse=None, stream=None):
        """``run`` merged by LSE with the state (prefix_out, prefix_lse) in the same
        call (mla_decode_suffix_merge). out/lse default to new tensors; passing
        prefix_out/prefix_lse themselves merges in place."""
        h = self.header()
        N, H = h.num_rows, self.num_heads
        if out is None:
            out = torch.empty_like(prefix_out)
        if lse is None:
            lse = torch.empty((N, H), dtype=torch.float32, device=self.device)
        assert q_nope.stride(-1) == 1 and q_rope.stride(-1) == 1
        stream = stream or torch.cuda.current_stream(self.device)
        st = B.mla_decode_suffix_merge(self.params, self.plan_h, self.workspace, self.workspace.numel(),
                                       q_nope, q_nope.stride(0), q_nope.stride(1), q_rope,
                                       q_rope.stride(0), q_rope.stride(1), kv_cache, kv_scale,
                                       kv_indices, kv_lens, sm_scale, prefix_out, prefix_lse, out,
                                       lse, stream)
        if st != B.MLA_OK:
            raise B.MlaError("mla_decode_suffix_merge", st)
        return out, lse


    def run_tree_verify(self, q_nope, q_rope, kv_cache, kv_indices, suffix_table, suffix_lens,
                        sm_scale, kv_scale=1.0, out=None, lse=None, stream=None):
        """Each planned row over its request's tokens and then its visible suffix
        slots (suffix_table [rows, stride] int32 pool rows, suffix_lens [rows]),
        in one pass (mla_decode_tree_verify). Needs suffix_tokens > 0."""
        h = self.header()
        N, H = h.num_rows, self.num_heads
        if out is None:
            dt = torch.float32 if self.out_dtype == "fp32" else torch.bfloat16
            out = torch.empty((N, H, 512), dtype=dt, device=self.device)
        if lse is None:
            lse = torch.empty((N, H), dtype=torch.float32, device=self.device)
        assert q_nope.stride(-1) == 1 and q_rope.stride(-1) == 1 and suffix_table.stride(-1) == 1
        stream = stream or torch.cuda.current_stream(self.device)
        st = B.mla_decode_tree_verify(self.params, self.plan_h, self.workspace, self.workspace.numel(),
                                      q_nope, q_nope.stride(0), q_nope.stride(1), q_rope,
                                      q_rope.stride(0), q_rope.stride(1), kv_cache, kv_scale,
                                      kv_indices, suffix_table, suffix_table.stride(0), suffix_lens,
                                      sm_scale, out, lse, stream)
        if st != B.MLA_OK:
            raise B.MlaError("mla_decode_tree_verify", st)
        return out, lse


def merge_states(v_a, s_a, v_b, s_b, out=None, s_out=None, stream=None):
    """LSE merge of two states (bf16 or fp32 v of shape [..., D], fp32 s of shape [...])."""
    assert v_a.dtype == v_b.dtype and v_a.shape == v_b.shape
    D = v_a.shape[-1]
    rows = v_a.numel() // D
    out = torch.empty_like(v_a) if out is None else out
    s_out = torch.empty_like(s_a) if s_out is None else s_out
    dt = B.MLA_DTYPE_FP32 if v_a.dtype == torch.float32 else B.MLA_DTYPE_BF16
    st = B.mla_merge_states(v_a, s_a, v_b, s_b, out, s_out, rows, D, dt,
                            stream or torch.cuda.current_stream(v_a.device))
    if st != B.MLA_OK:
        raise B.MlaError("mla_merge_states", st)
    return out, s_out


def tree_suffix_compact(tree_mask, req_to_token, prefix_lens, width, num_rows=None,
                        num_actual_rows=None, stream=None):
    """(page_table [rows, width] int32, cache_seqlens [rows] int32) on the device."""
    n_actual = tree_mask.shape[0] if num_actual_rows is None else int(num_actual_rows)
    rows = n_actual if num_rows is None else int(num_rows)
    dev = req_to_token.device
    table = torch.empty((rows, width), dtype=torch.int32, device=dev)
    seqlens = torch.empty(rows, dtype=torch.int32, device=dev)
    st = B.mla_tree_suffix_compact(tree_mask, tree_mask.stride(0), req_to_token,
                                   req_to_token.stride(0), prefix_lens, width, rows, n_actual,
                                   table, table.stride(0), seqlens,
                                   stream or torch.cuda.current_stream(dev))
    if st != B.MLA_OK:
        raise B.MlaError("mla_tree_suffix_compact", st)
    return table, seqlens


def absorb_query(q, w_uk, out=None, stream=None):
    """q [N, H, D] bf16 (D contiguous), w_uk [512, H, D] or any strided view with D
    contiguous, indexed (a, h, d) -> q_abs [N, H, 512] bf16 (or written into `out`,
    e.g. the first 512 columns of a [N, H, 576] query)."""
    N, H, D = q.shape
    assert w_uk.shape == (512, H, D) and q.stride(2) == 1 and w_uk.stride(2) == 1
    out = torch.empty((N, H, 512), dtype=torch.bfloat16, device=q.device) if out is None else out
    assert out.shape == (N, H, 512) and out.stride(2) == 1
    st = B.mla_absorb_query(q, q.stride(0), q.stride(1), w_uk, w_uk.stride(0), w_uk.stride(1),
                            out, out.stride(0), out.stride(1), N, H, D,
                            stream or torch.cuda.current_stream(q.device))
    if st != B.MLA_OK:
        raise B.MlaError("mla_absorb_query", st)
    return out


def project_output(x, w_uv, out=None, stream=None):
    """x [N, H, 512] bf16 (latent contiguous), w_uv any view indexed (a, h, d) with a
    contiguous (e.g. kv_b_proj's value rows viewed as [512, H, D]) -> o [N, H, D] bf16."""
    N, H, A = x.shape
    D = w_uv.shape[2]
    assert A == 512 and w_uv.shape == (512, H, D) and x.stride(2) == 1 and w_uv.stride(0) == 1
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device=x.device) if out is None else out
    assert out.shape == (N, H, D) and out.stride(2) == 1
    st = B.mla_project_output(x, x.stride(0), x.stride(1), w_uv, w_uv.stride(1), w_uv.stride(2),
                              out, out.stride(0), out.stride(1), N, H, D,
                              stream or torch.cuda.current_stream(x.device))
    if st != B.MLA_OK:
        raise B.MlaError("mla_project_output", st)
    return out
