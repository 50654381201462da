"""Weight-absorbed MLA decode over a paged latent KV cache, for MI355X (gfx950).

The computation lives in libmla_decode.so (hand-written HIP kernels and a C++
host planner, C ABI in include/mla_decode.h). This package is its thin binding:
``_binding`` mirrors the C entry points one for one, ``decoder`` adds buffer
management with torch allocations, ``costs`` is the host-side cost model.

Names load on first use: importing the package (for instance to run its
``build`` module before the library exists) loads nothing. The first use of
a binding name loads the library, and raises if it is not built: there is no
fallback implementation.
"""

_BINDING = (
    "EXPORTED_SYMBOLS", "LIB_PATH", "MLA_DTYPE_BF16", "MLA_DTYPE_FP8_E4M3FN", "MLA_DTYPE_FP32",
    "MLA_ERR_HIP", "MLA_ERR_INVALID_ARG", "MLA_ERR_PLAN_MISMATCH", "MLA_ERR_UNSUPPORTED",
    "MLA_ERR_WORKSPACE_TOO_SMALL", "MLA_ITEM_LAST_CHUNK", "MLA_DECODE_GRAPH_SAFE", "MLA_DECODE_FP8_SCORE", "MLA_DECODE_SHARED_ROWS", "MLA_OK",
    "MLA_PLAN_VERSION", "MlaError",
    "make_params", "mla_absorb_query", "mla_decode", "mla_decode_append", "mla_decode_plan",
    "mla_decode_suffix_merge", "mla_decode_tree_verify", "mla_decode_variant",
    "mla_decode_workspace_size",
    "mla_merge_states", "mla_project_output", "mla_status_string", "mla_tree_suffix_compact",
    "read_plan")
# torch-based helpers, so that the host-only ABI can be used without a GPU.
_DECODER = ("PagedMlaDecoder", "merge_states", "tree_suffix_compact", "absorb_query",
            "project_output")

__all__ = list(_BINDING + _DECODER)


def __getattr__(name):
    if name in _BINDING:
        from . import _binding
        return getattr(_binding, name)
    if name in _DECODER:
        from . import decoder
        return getattr(decoder, name)
    raise AttributeError(name)


def __dir__():
    return sorted(list(globals()) + __all__)
