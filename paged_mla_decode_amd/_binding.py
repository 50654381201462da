"""ctypes binding of libmla_decode.so (see include/mla_decode.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels or its host planner. Device buffers are passed as raw pointers;
torch tensors are accepted for convenience (their data_ptr() is passed) and
torch is otherwise only used by callers for memory and streams.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m paged_mla_decode_amd.build` "
        "(hipcc for gfx950). There is no fallback implementation.")

# One HIP runtime per process: torch's wheel bundles its own libamdhip64 (SONAME
# libamdhip64.so.7) and loads it by an unversioned name. Loading torch first
# lets this library's libamdhip64.so.7 dependency bind to that same runtime, so
# torch's device pointers and streams are valid here. Loaded the other way
# round, the process would hold two HIP runtimes.
try:
    import torch  # noqa: F401
except ImportError:  # the library itself does not need torch
    torch = None

_lib = ctypes.CDLL(LIB_PATH)

# ---- constants (mla_decode.h) ----
MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_ERR_PLAN_MISMATCH = 5
MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP32 = 1
MLA_DTYPE_FP8_E4M3FN = 2
MLA_PLAN_MAGIC = 0x504C4D41
MLA_PLAN_VERSION = 7
MLA_DECODE_GRAPH_SAFE = 1
MLA_DECODE_FP8_SCORE = 2
MLA_DECODE_SHARED_ROWS = 4
MLA_ITEM_LAST_CHUNK = 1


class mla_decode_params(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_rope_head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("suffix_tokens", ctypes.c_int32)]


class mla_plan_header(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("num_items", ctypes.c_int32), ("num_merges", ctypes.c_int32),
                ("num_partials", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("num_workers", ctypes.c_int32), ("max_merge_partials", ctypes.c_int32),
                ("num_wide_merges", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("suffix_tokens", ctypes.c_int32), ("tiles_read_once", ctypes.c_int32),
                ("num_page_entries", ctypes.c_int64), ("items_offset", ctypes.c_int64),
                ("merges_offset", ctypes.c_int64), ("workers_offset", ctypes.c_int64),
                ("plan_bytes", ctypes.c_int64),
                ("partial_out_offset", ctypes.c_int64), ("partial_lse_offset", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64),
                ("query_codes_offset", ctypes.c_int64), ("query_exp_offset", ctypes.c_int64)]


class mla_work_item(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("row", "request", "page_base", "kv_begin", "kv_end", "partial", "head_begin")] + \
        [("flags", ctypes.c_uint32), ("num_rows", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class mla_merge_item(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("row", "partial_begin", "num_partials", "partial_stride")]


_p = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_PARAMS = ctypes.POINTER(mla_decode_params)

_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_status_string.argtypes = [_i32]
_lib.mla_decode_variant.restype = ctypes.c_char_p
_lib.mla_decode_variant.argtypes = [_PARAMS]
_lib.mla_decode_workspace_size.restype = _i32
_lib.mla_decode_workspace_size.argtypes = [_PARAMS, _i32, _i32, ctypes.POINTER(_sz),
                                           ctypes.POINTER(_sz)]
_lib.mla_decode_plan.restype = _i32
_lib.mla_decode_plan.argtypes = [_PARAMS, _i32, _p, _p, _p, _p, _sz, _p, _sz, _p]
_lib.mla_decode.restype = _i32
_lib.mla_decode.argtypes = [_PARAMS, _p, _p, _sz, _p, _i64, _i64, _p, _i64, _i64, _p, _f32, _p,
                            _p, _f32, _p, _p, _p]
_lib.mla_decode_noalloc.restype = _i32
_lib.mla_decode_noalloc.argtypes = [_PARAMS, _p, _p, _i64, _i64, _p, _i64, _i64, _p, _f32, _p, _p, _f32,
                                    _p, _p, _p]
_lib.mla_decode_append.restype = _i32
_lib.mla_decode_append.argtypes = [_PARAMS, _p, _p, _sz, _p, _i64, _i64, _p, _i64, _i64, _p, _f32,
                                   _p, _p, _i64, _p, _i64, _f32, _p, _p, _p]
_lib.mla_decode_suffix_merge.restype = _i32
_lib.mla_decode_suffix_merge.argtypes = [_PARAMS, _p, _p, _sz, _p, _i64, _i64, _p, _i64, _i64, _p,
                                         _f32, _p, _p, _f32, _p, _p, _p, _p, _p]
_lib.mla_decode_tree_verify.restype = _i32
_lib.mla_decode_tree_verify.argtypes = [_PARAMS, _p, _p, _sz, _p, _i64, _i64, _p, _i64, _i64, _p,
                                        _f32, _p, _p, _i64, _p, _f32, _p, _p, _p]
_lib.mla_merge_states.restype = _i32
_lib.mla_merge_states.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _p]
_lib.mla_tree_suffix_compact.restype = _i32
_lib.mla_tree_suffix_compact.argtypes = [_p, _i64, _p, _i64, _p, _i32, _i32, _i32, _p, _i64, _p,
                                         _p]
for _fn in (_lib.mla_absorb_query, _lib.mla_project_output):
    _fn.restype = _i32
    _fn.argtypes = [_p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i32, _i32, _i32, _p]
_PI64 = ctypes.POINTER(_i64)
_lib.mla_decode_validate_batch.restype = _i32
_lib.mla_decode_validate_batch.argtypes = [_i32, _i32, _p, _p, _p, _p, _i64, _PI64]
_lib.mla_tree_validate_inputs.restype = _i32
_lib.mla_tree_validate_inputs.argtypes = [_p, _i64, _i32, _p, _i32, _i64, _PI64]
_lib.mla_tree_validate_suffix.restype = _i32
_lib.mla_tree_validate_suffix.argtypes = [_p, _i64, _p, _i32, _i32, _i64, _PI64]

EXPORTED_SYMBOLS = ("mla_status_string", "mla_decode_variant", "mla_decode_workspace_size",
                    "mla_decode_plan", "mla_decode", "mla_decode_append", "mla_decode_suffix_merge",
                    "mla_decode_tree_verify",
                    "mla_merge_states",
                    "mla_tree_suffix_compact", "mla_absorb_query", "mla_project_output",
                    "mla_decode_validate_batch", "mla_tree_validate_inputs",
                    "mla_tree_validate_suffix", "mla_decode_noalloc")


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {mla_status_string(status)} ({status})")


def _ptr(x):
    """A device or host pointer from a torch tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take a pointer of {type(x)}")


def _stream(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != MLA_OK:
        raise MlaError(fn, status)


def make_params(num_heads, page_size, kv_dtype=MLA_DTYPE_BF16, out_dtype=MLA_DTYPE_BF16,
                num_cus=0, max_splits=0, kv_lora_rank=512, qk_rope_head_dim=64, flags=0,
                max_rows=0, suffix_tokens=0):
    return mla_decode_params(num_heads, kv_lora_rank, qk_rope_head_dim, page_size, kv_dtype,
                             out_dtype, num_cus, max_splits, flags, max_rows, suffix_tokens)


# ---- the C-ABI entry points, same names ----

def mla_status_string(status: int) -> str:
    return _lib.mla_status_string(int(status)).decode()


def mla_decode_variant(params: mla_decode_params):
    r = _lib.mla_decode_variant(ctypes.byref(params))
    return None if r is None else r.decode()


def mla_decode_workspace_size(params, batch, num_rows):
    pb, wb = _sz(0), _sz(0)
    _check("mla_decode_workspace_size",
           _lib.mla_decode_workspace_size(ctypes.byref(params), int(batch), int(num_rows),
                                          ctypes.byref(pb), ctypes.byref(wb)))
    return pb.value, wb.value


def mla_decode_plan(params, batch, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, plan_h,
                    plan_h_bytes, workspace_d=None, workspace_bytes=0, stream=None):
    """Returns the status code (raises nothing), so callers can test error paths."""
    return _lib.mla_decode_plan(ctypes.byref(params), int(batch), _ptr(qo_indptr_h),
                                _ptr(kv_indptr_h), _ptr(kv_last_page_len_h), _ptr(plan_h),
                                int(plan_h_bytes), _ptr(workspace_d), int(workspace_bytes),
                                _stream(stream) if workspace_d is not None else None)


def mla_decode(params, plan_h, workspace_d, workspace_bytes, q_nope_d, q_nope_stride_n,
               q_nope_stride_h, q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d, kv_scale,
               kv_indices_d, kv_lens_d, sm_scale, out_d, lse_d, stream=None):
    return _lib.mla_decode(ctypes.byref(params), _ptr(plan_h), _ptr(workspace_d),
                           int(workspace_bytes), _ptr(q_nope_d), int(q_nope_stride_n),
                           int(q_nope_stride_h), _ptr(q_rope_d), int(q_rope_stride_n),
                           int(q_rope_stride_h), _ptr(kv_cache_d), float(kv_scale),
                           _ptr(kv_indices_d), _ptr(kv_lens_d), float(sm_scale), _ptr(out_d),
                           _ptr(lse_d), _stream(stream))


def mla_decode_noalloc(params, plan_h, q_nope_d, q_nope_stride_n, q_nope_stride_h, q_rope_d,
                       q_rope_stride_n, q_rope_stride_h, kv_cache_d, kv_scale, kv_indices_d,
                       kv_lens_d, sm_scale, out_d, lse_d, stream=None):
    return _lib.mla_decode_noalloc(ctypes.byref(params), _ptr(plan_h), _ptr(q_nope_d),
                                   int(q_nope_stride_n), int(q_nope_stride_h), _ptr(q_rope_d),
                                   int(q_rope_stride_n), int(q_rope_stride_h), _ptr(kv_cache_d),
                                   float(kv_scale), _ptr(kv_indices_d), _ptr(kv_lens_d),
                                   float(sm_scale), _ptr(out_d), _ptr(lse_d), _stream(stream))


def mla_decode_append(params, plan_h, workspace_d, workspace_bytes, q_nope_d, q_nope_stride_n,
                      q_nope_stride_h, q_rope_d, q_rope_stride_n, q_rope_stride_h, kv_cache_d,
                      kv_scale, kv_indices_d, c_new_d, c_new_stride, k_pe_new_d, k_pe_new_stride,
                      sm_scale, out_d, lse_d, stream=None):
    return _lib.mla_decode_append(ctypes.byref(params), _ptr(plan_h), _ptr(workspace_d),
                                  int(workspace_bytes), _ptr(q_nope_d), int(q_nope_stride_n),
                                  int(q_nope_stride_h), _ptr(q_rope_d), int(q_rope_stride_n),
                                  int(q_rope_stride_h), _ptr(kv_cache_d), float(kv_scale),
                                  _ptr(kv_indices_d), _ptr(c_new_d), int(c_new_stride),
                                  _ptr(k_pe_new_d), int(k_pe_new_stride), float(sm_scale),
                                  _ptr(out_d), _ptr(lse_d), _stream(stream))


def mla_decode_suffix_merge(params, plan_h, workspace_d, workspace_bytes, q_nope_d,
                            q_nope_stride_n, q_nope_stride_h, q_rope_d, q_rope_stride_n,
                            q_rope_stride_h, kv_cache_d, kv_scale, kv_indices_d, kv_lens_d,
                            sm_scale, prefix_out_d, prefix_lse_d, out_d, lse_d, stream=None):
    return _lib.mla_decode_suffix_merge(
        ctypes.byref(params), _ptr(plan_h), _ptr(workspace_d), int(workspace_bytes), _ptr(q_nope_d),
        int(q_nope_stride_n), int(q_nope_stride_h), _ptr(q_rope_d), int(q_rope_stride_n),
        int(q_rope_stride_h), _ptr(kv_cache_d), float(kv_scale), _ptr(kv_indices_d), _ptr(kv_lens_d),
        float(sm_scale), _ptr(prefix_out_d), _ptr(prefix_lse_d), _ptr(out_d), _ptr(lse_d),
        _stream(stream))


def mla_decode_tree_verify(params, plan_h, workspace_d, workspace_bytes, q_nope_d,
                           q_nope_stride_n, q_nope_stride_h, q_rope_d, q_rope_stride_n,
                           q_rope_stride_h, kv_cache_d, kv_scale, kv_indices_d, suffix_table_d,
                           suffix_stride, suffix_lens_d, sm_scale, out_d, lse_d, stream=None):
    return _lib.mla_decode_tree_verify(
        ctypes.byref(params), _ptr(plan_h), _ptr(workspace_d), int(workspace_bytes), _ptr(q_nope_d),
        int(q_nope_stride_n), int(q_nope_stride_h), _ptr(q_rope_d), int(q_rope_stride_n),
        int(q_rope_stride_h), _ptr(kv_cache_d), float(kv_scale), _ptr(kv_indices_d),
        _ptr(suffix_table_d), int(suffix_stride), _ptr(suffix_lens_d), float(sm_scale), _ptr(out_d),
        _ptr(lse_d), _stream(stream))


def mla_merge_states(v_a_d, s_a_d, v_b_d, s_b_d, v_out_d, s_out_d, num_rows, head_dim, v_dtype,
                     stream=None):
    return _lib.mla_merge_states(_ptr(v_a_d), _ptr(s_a_d), _ptr(v_b_d), _ptr(s_b_d),
                                 _ptr(v_out_d), _ptr(s_out_d), int(num_rows), int(head_dim),
                                 int(v_dtype), _stream(stream))


def mla_tree_suffix_compact(tree_mask_d, mask_stride, req_to_token_d, req_stride, prefix_lens_d,
                            width, num_rows, num_actual_rows, page_table_d, table_stride,
                            cache_seqlens_d, stream=None):
    return _lib.mla_tree_suffix_compact(_ptr(tree_mask_d), int(mask_stride), _ptr(req_to_token_d),
                                        int(req_stride), _ptr(prefix_lens_d), int(width),
                                        int(num_rows), int(num_actual_rows), _ptr(page_table_d),
                                        int(table_stride), _ptr(cache_seqlens_d),
                                        _stream(stream))


def mla_absorb_query(q_d, q_stride_n, q_stride_h, w_uk_d, w_uk_stride_a, w_uk_stride_h, q_abs_d,
                     q_abs_stride_n, q_abs_stride_h, num_rows, num_heads, head_dim, stream=None):
    return _lib.mla_absorb_query(_ptr(q_d), int(q_stride_n), int(q_stride_h), _ptr(w_uk_d),
                                 int(w_uk_stride_a), int(w_uk_stride_h), _ptr(q_abs_d),
                                 int(q_abs_stride_n), int(q_abs_stride_h), int(num_rows),
                                 int(num_heads), int(head_dim), _stream(stream))


def mla_project_output(x_d, x_stride_n, x_stride_h, w_uv_d, w_uv_stride_h, w_uv_stride_d, o_d,
                       o_stride_n, o_stride_h, num_rows, num_heads, head_dim, stream=None):
    return _lib.mla_project_output(_ptr(x_d), int(x_stride_n), int(x_stride_h), _ptr(w_uv_d),
                                   int(w_uv_stride_h), int(w_uv_stride_d), _ptr(o_d),
                                   int(o_stride_n), int(o_stride_h), int(num_rows),
                                   int(num_heads), int(head_dim), _stream(stream))


def read_plan(plan_h):
    """(header, [work items], [merge items], [worker item offsets]) copied out of a
    host plan buffer."""
    base = _ptr(plan_h)
    h = mla_plan_header.from_buffer_copy(ctypes.string_at(base, ctypes.sizeof(mla_plan_header)))
    items = (mla_work_item * h.num_items).from_buffer_copy(
        ctypes.string_at(base + h.items_offset, h.num_items * ctypes.sizeof(mla_work_item)))
    merges = (mla_merge_item * h.num_merges).from_buffer_copy(
        ctypes.string_at(base + h.merges_offset, h.num_merges * ctypes.sizeof(mla_merge_item)))
    workers = (ctypes.c_int32 * (h.num_workers + 1)).from_buffer_copy(
        ctypes.string_at(base + h.workers_offset, (h.num_workers + 1) * 4))
    return h, list(items), list(merges), list(workers)


# ---- host checks of index arrays against the pool ----
# Each takes host arrays (numpy int32, C-contiguous) and returns
# (status, bad_entry): the first offending entry's index, or -1.

def mla_decode_validate_batch(page_size, batch, qo_indptr_h, kv_indptr_h, kv_indices_h,
                              kv_last_page_len_h, num_pool_pages):
    bad = _i64(-1)
    st = _lib.mla_decode_validate_batch(int(page_size), int(batch), _ptr(qo_indptr_h),
                                        _ptr(kv_indptr_h), _ptr(kv_indices_h),
                                        _ptr(kv_last_page_len_h), int(num_pool_pages),
                                        ctypes.byref(bad))
    return st, bad.value


def mla_tree_validate_inputs(req_to_token_h, req_stride, num_requests, prefix_lens_h, width,
                             num_pool_rows):
    bad = _i64(-1)
    st = _lib.mla_tree_validate_inputs(_ptr(req_to_token_h), int(req_stride), int(num_requests),
                                       _ptr(prefix_lens_h), int(width), int(num_pool_rows),
                                       ctypes.byref(bad))
    return st, bad.value


def mla_tree_validate_suffix(suffix_table_h, suffix_stride, suffix_lens_h, num_rows, suffix_tokens,
                             num_pool_rows):
    bad = _i64(-1)
    st = _lib.mla_tree_validate_suffix(_ptr(suffix_table_h), int(suffix_stride), _ptr(suffix_lens_h),
                                       int(num_rows), int(suffix_tokens), int(num_pool_rows),
                                       ctypes.byref(bad))
    return st, bad.value
