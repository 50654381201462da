"""C-ABI library: loads, exports every declared symbol, and rejects bad
arguments on the host with its documented status codes (no GPU work)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import paged_mla_decode_amd as m
from paged_mla_decode_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")
FAKE = 1 << 40  # a non-null, 16-byte aligned stand-in address; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|int32_t)\s+(mla_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 16
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED_SYMBOLS) == names


def test_struct_layouts_match_header(tmp_path):
    """The binding's ctypes structs have the C header's size and field offsets
    (checked against the host compiler's view of include/mla_decode.h)."""
    structs = [B.mla_decode_params, B.mla_plan_header, B.mla_work_item, B.mla_merge_item]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mla_decode.h"', 'int main(void) {']
    for st in structs:
        lines.append(f'printf("{st.__name__} %zu\\n", sizeof({st.__name__}));')
        for name, _ in st._fields_:
            lines.append(f'printf("{st.__name__}.{name} %zu\\n", offsetof({st.__name__}, {name}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)], text=True).splitlines())
    for st in structs:
        assert int(got[st.__name__]) == ctypes.sizeof(st), st.__name__
        for name, _ in st._fields_:
            assert int(got[f"{st.__name__}.{name}"]) == getattr(st, name).offset, (st.__name__, name)


def test_status_strings():
    assert m.mla_status_string(0) == "MLA_OK"
    assert m.mla_status_string(5) == "MLA_ERR_PLAN_MISMATCH"
    assert m.mla_status_string(99) == "MLA_ERR_UNKNOWN"


@pytest.mark.parametrize("H,variant", [(16, "hw16,hs2"), (32, "hw16,hs2"), (64, "hw16,hs4"),
                                       (128, "hw32,hs4")])
def test_variant_names(H, variant):
    p = m.make_params(H, 1, num_cus=256)
    assert variant in m.mla_decode_variant(p)
    p8 = m.make_params(H, 64, kv_dtype=m.MLA_DTYPE_FP8_E4M3FN, out_dtype=m.MLA_DTYPE_FP32,
                       num_cus=256)
    assert m.mla_decode_variant(p8).endswith("kv_fp8,out_fp32>")


@pytest.mark.parametrize("bad", [
    dict(num_heads=48), dict(num_heads=256), dict(kv_lora_rank=256), dict(qk_rope_head_dim=128),
    dict(page_size=0), dict(kv_dtype=1), dict(out_dtype=2)])
def test_unsupported_params(bad):
    kw = dict(num_heads=128, page_size=64, num_cus=256)
    kw.update(bad)
    p = m.make_params(**kw)
    assert m.mla_decode_variant(p) is None
    plan = np.zeros(1 << 16, np.uint8)
    st = m.mla_decode_plan(p, 1, None, np.array([0, 1], np.int32), None, plan, plan.size)
    assert st in (m.MLA_ERR_UNSUPPORTED, m.MLA_ERR_INVALID_ARG)


def _plan(p, kv_indptr, last=None, qo=None, size=1 << 20):
    plan = np.zeros(size, np.uint8)
    qo = None if qo is None else np.asarray(qo, np.int32)
    st = m.mla_decode_plan(p, len(kv_indptr) - 1, qo, np.asarray(kv_indptr, np.int32),
                           None if last is None else np.asarray(last, np.int32), plan, size)
    return st, plan


def test_plan_rejects_malformed_csr():
    p = m.make_params(16, 4, num_cus=256)
    assert _plan(p, [0, 3, 2])[0] == m.MLA_ERR_INVALID_ARG  # decreasing indptr
    assert _plan(p, [-1, 2])[0] == m.MLA_ERR_INVALID_ARG
    assert _plan(p, [0, 2, 3], last=[0, 1])[0] == m.MLA_ERR_INVALID_ARG  # last_page_len < 1
    assert _plan(p, [0, 2, 3], last=[5, 1])[0] == m.MLA_ERR_INVALID_ARG  # > page_size
    assert _plan(p, [0, 2, 3], qo=[1, 2, 3])[0] == m.MLA_ERR_INVALID_ARG  # qo_indptr[0] != 0
    assert _plan(p, [0, 2, 3], qo=[0, 2, 1])[0] == m.MLA_ERR_INVALID_ARG
    assert m.mla_decode_plan(p, 1, None, None, None, np.zeros(64, np.uint8), 64) == \
        m.MLA_ERR_INVALID_ARG
    assert _plan(p, [0, 2, 3], last=[4, 1])[0] == m.MLA_OK


def test_plan_buffer_too_small():
    p = m.make_params(16, 1, num_cus=256)
    st, _ = _plan(p, [0, 100, 200], size=64)
    assert st == m.MLA_ERR_WORKSPACE_TOO_SMALL


def test_workspace_bounds_cover_actual_plans():
    rng = np.random.default_rng(0)
    for H in (16, 128):
        p = m.make_params(H, 16, num_cus=256)
        for _ in range(20):
            B_ = int(rng.integers(1, 40))
            npages = rng.integers(0, 400, size=B_)
            indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
            last = np.where(npages > 0, rng.integers(1, 17, size=B_), 1)
            pb, wb = m.mla_decode_workspace_size(p, B_, B_)
            st, plan = _plan(p, indptr, last, size=pb)
            assert st == m.MLA_OK
            h = m.read_plan(plan)[0]
            assert h.plan_bytes <= pb and h.workspace_bytes <= wb


def test_decode_validates_before_launch():
    p = m.make_params(16, 1, num_cus=256)
    st, plan = _plan(p, [0, 5])
    h = m.read_plan(plan)[0]
    ws = h.workspace_bytes

    def call(**over):
        args = dict(params=p, plan_h=plan, workspace_d=FAKE, workspace_bytes=ws, q_nope_d=FAKE,
                    q_nope_stride_n=16 * 512, q_nope_stride_h=512, q_rope_d=FAKE,
                    q_rope_stride_n=16 * 64, q_rope_stride_h=64, kv_cache_d=FAKE, kv_scale=1.0,
                    kv_indices_d=FAKE, kv_lens_d=None, sm_scale=0.1, out_d=FAKE, lse_d=None,
                    stream=0)
        args.update(over)
        return m.mla_decode(**args)

    assert call(q_nope_d=None) == m.MLA_ERR_INVALID_ARG
    assert call(kv_cache_d=None) == m.MLA_ERR_INVALID_ARG
    assert call(kv_indices_d=None) == m.MLA_ERR_INVALID_ARG  # the batch has page entries
    assert call(out_d=FAKE + 8) == m.MLA_ERR_INVALID_ARG  # misaligned
    assert call(q_nope_stride_h=500) == m.MLA_ERR_INVALID_ARG
    assert call(sm_scale=float("nan")) == m.MLA_ERR_INVALID_ARG
    assert call(sm_scale=0.0) == m.MLA_ERR_INVALID_ARG
    assert call(sm_scale=-0.1) == m.MLA_ERR_INVALID_ARG
    assert call(kv_scale=2.0) == m.MLA_ERR_INVALID_ARG  # bf16 cache takes no scale
    assert call(workspace_bytes=ws - 1) == m.MLA_ERR_WORKSPACE_TOO_SMALL
    other = m.make_params(32, 1, num_cus=256)
    assert call(params=other) == m.MLA_ERR_PLAN_MISMATCH
    bad = plan.copy()
    bad[:4] = 0
    assert call(plan_h=bad) == m.MLA_ERR_INVALID_ARG


def test_decode_append_validates_before_launch():
    """Every check runs on the host; the fake device pointers are never touched."""
    p = m.make_params(16, 1, num_cus=256)

    def call(plan, **over):
        h = m.read_plan(plan)[0]
        args = dict(params=p, plan_h=plan, workspace_d=FAKE, workspace_bytes=h.workspace_bytes,
                    q_nope_d=FAKE, q_nope_stride_n=16 * 512, q_nope_stride_h=512, q_rope_d=FAKE,
                    q_rope_stride_n=16 * 64, q_rope_stride_h=64, kv_cache_d=FAKE, kv_scale=1.0,
                    kv_indices_d=FAKE, c_new_d=FAKE, c_new_stride=576, k_pe_new_d=FAKE + 1024,
                    k_pe_new_stride=576, sm_scale=0.1, out_d=FAKE, lse_d=None, stream=0)
        args.update(over)
        return m.mla_decode_append(**args)

    st, empty_req = _plan(p, [0, 0, 5])  # request 0 has no token to hold the new one
    assert st == m.MLA_OK
    assert call(empty_req) == m.MLA_ERR_INVALID_ARG
    st, good = _plan(p, [0, 3, 8])
    assert st == m.MLA_OK
    assert call(good, c_new_d=None) == m.MLA_ERR_INVALID_ARG
    assert call(good, k_pe_new_d=FAKE + 8) == m.MLA_ERR_INVALID_ARG
    assert call(good, c_new_stride=570) == m.MLA_ERR_INVALID_ARG
    assert call(good, k_pe_new_stride=-8) == m.MLA_ERR_INVALID_ARG
    assert call(good, sm_scale=0.0) == m.MLA_ERR_INVALID_ARG
    # Two query rows on one request: one new token per request is not defined.
    pb, _ = m.mla_decode_workspace_size(p, 2, 3)
    plan2 = np.zeros(pb, dtype=np.uint8)
    assert m.mla_decode_plan(p, 2, np.array([0, 2, 3], np.int32), np.array([0, 3, 8], np.int32),
                             None, plan2, pb) == m.MLA_OK
    assert call(plan2) == m.MLA_ERR_INVALID_ARG


def test_tree_verify_plans_only_reach_the_tree_call():
    p = m.make_params(128, 1, num_cus=16, suffix_tokens=8)
    st, plan = _plan(p, [0, 40, 90])
    assert st == m.MLA_OK
    h = m.read_plan(plan)[0]
    common = dict(params=p, plan_h=plan, workspace_d=FAKE, workspace_bytes=h.workspace_bytes,
                  q_nope_d=FAKE, q_nope_stride_n=128 * 512, q_nope_stride_h=512, q_rope_d=FAKE,
                  q_rope_stride_n=128 * 64, q_rope_stride_h=64, kv_cache_d=FAKE, kv_scale=1.0,
                  kv_indices_d=FAKE, sm_scale=0.1, out_d=FAKE, lse_d=None, stream=0)
    assert m.mla_decode(kv_lens_d=None, **common) == m.MLA_ERR_INVALID_ARG
    tree = dict(suffix_table_d=FAKE, suffix_stride=64, suffix_lens_d=FAKE)
    assert m.mla_decode_tree_verify(**{**common, **tree, "suffix_table_d": None}) == m.MLA_ERR_INVALID_ARG
    assert m.mla_decode_tree_verify(**{**common, **tree, "suffix_stride": 4}) == m.MLA_ERR_INVALID_ARG
    plain = m.make_params(128, 1, num_cus=16)
    assert m.mla_decode_tree_verify(**{**common, **tree, "params": plain}) == m.MLA_ERR_PLAN_MISMATCH


def test_merge_and_compact_validate():
    assert m.mla_merge_states(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 7, 0, 0) == m.MLA_ERR_INVALID_ARG
    assert m.mla_merge_states(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 2, 0) == \
        m.MLA_ERR_UNSUPPORTED
    assert m.mla_merge_states(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8192, 0, 0) == \
        m.MLA_ERR_UNSUPPORTED
    assert m.mla_merge_states(None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 0, 0) == \
        m.MLA_ERR_INVALID_ARG
    assert m.mla_merge_states(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 512, 0, 0) == m.MLA_OK
    c = m.mla_tree_suffix_compact
    assert c(FAKE, 64, FAKE, 80, FAKE, 0, 8, 8, FAKE, 64, FAKE, 0) == m.MLA_ERR_INVALID_ARG
    assert c(FAKE, 2048, FAKE, 2048, FAKE, 2000, 8, 8, FAKE, 2048, FAKE, 0) == m.MLA_ERR_UNSUPPORTED
    assert c(FAKE, 64, FAKE, 80, FAKE, 64, 8, 9, FAKE, 64, FAKE, 0) == m.MLA_ERR_INVALID_ARG
    assert c(FAKE, 64, FAKE, 80, FAKE, 64, 8, 8, FAKE, 32, FAKE, 0) == m.MLA_ERR_INVALID_ARG
    assert c(FAKE, 32, FAKE, 80, FAKE, 64, 8, 8, FAKE, 64, FAKE, 0) == m.MLA_ERR_INVALID_ARG
    assert c(None, 64, FAKE, 80, FAKE, 64, 8, 8, FAKE, 64, FAKE, 0) == m.MLA_ERR_INVALID_ARG
    assert c(FAKE, 64, FAKE, 80, FAKE, 64, 0, 0, FAKE, 64, FAKE, 0) == m.MLA_OK


@pytest.mark.parametrize("fn", ["mla_absorb_query", "mla_project_output"])
def test_projections_validate(fn):
    f = getattr(m, fn)
    # (x, xn, xh, w, w0, w1, y, yn, yh, rows, heads, head_dim, stream)
    good = [FAKE, 128 * 128, 128, FAKE, 128 * 128, 128, FAKE, 128 * 512, 512, 4, 128, 128, 0]

    def call(**kw):
        a = list(good)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)

    assert call(a9=0) == m.MLA_OK  # nothing to do: no launch
    assert call(a9=-1) == m.MLA_ERR_INVALID_ARG
    assert call(a10=0) == m.MLA_ERR_INVALID_ARG
    assert call(a11=64) == m.MLA_ERR_UNSUPPORTED
    assert call(a11=0) == m.MLA_ERR_INVALID_ARG
    assert call(a9=32 * 65535 + 1) == m.MLA_ERR_UNSUPPORTED
    assert call(a10=65536) == m.MLA_ERR_UNSUPPORTED
    for i in (0, 3, 6):
        assert call(**{f"a{i}": None}) == m.MLA_ERR_INVALID_ARG
        assert call(**{f"a{i}": FAKE + 8}) == m.MLA_ERR_INVALID_ARG  # 8-byte aligned only
    for i in (1, 2, 4, 5, 7, 8):
        assert call(**{f"a{i}": 12}) == m.MLA_ERR_INVALID_ARG
        assert call(**{f"a{i}": -8}) == m.MLA_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# The fp8 score flag (MLA_DECODE_FP8_SCORE)
# ---------------------------------------------------------------------------

def _qf8_params(**over):
    kw = dict(num_heads=128, page_size=64, kv_dtype=m.MLA_DTYPE_FP8_E4M3FN, num_cus=256,
              flags=m.MLA_DECODE_FP8_SCORE)
    kw.update(over)
    return m.make_params(**kw)


def test_fp8_score_only_for_the_128_head_fp8_bf16_plain_decode():
    assert m.mla_decode_variant(_qf8_params()).endswith("score_fp8>")
    for bad in (dict(num_heads=16), dict(num_heads=64), dict(kv_dtype=m.MLA_DTYPE_BF16),
                dict(out_dtype=m.MLA_DTYPE_FP32), dict(page_size=1, suffix_tokens=8)):
        assert m.mla_decode_variant(_qf8_params(**bad)) is None, bad
    assert m.mla_decode_variant(_qf8_params(flags=8)) is None  # an unknown flag


@pytest.mark.parametrize("graph", [False, True])
def test_fp8_score_workspace_holds_the_quantised_query(graph):
    flags = m.MLA_DECODE_FP8_SCORE | (m.MLA_DECODE_GRAPH_SAFE if graph else 0)
    p = _qf8_params(flags=flags, max_rows=40 if graph else 0)
    plain = m.make_params(128, 64, kv_dtype=m.MLA_DTYPE_FP8_E4M3FN, num_cus=256,
                          flags=m.MLA_DECODE_GRAPH_SAFE if graph else 0, max_rows=40 if graph else 0)
    indptr = [0, 3, 50, 51]
    pb, wb = m.mla_decode_workspace_size(p, 3, 3)
    st, plan = _plan(p, indptr, size=pb)
    assert st == m.MLA_OK
    h = m.read_plan(plan)[0]
    rows = 40 if graph else 3
    assert h.query_codes_offset >= h.partial_lse_offset + h.num_partials * 128 * 4 or h.num_partials == 0
    assert h.query_codes_offset % 256 == 0 and h.query_exp_offset % 256 == 0
    assert h.query_exp_offset >= h.query_codes_offset + rows * 128 * 576
    assert h.workspace_bytes >= h.query_exp_offset + rows * 128 * 4
    assert h.workspace_bytes <= wb
    # Without the flag the regions are absent and everything else sits where it did.
    st, plan0 = _plan(plain, indptr)
    h0 = m.read_plan(plan0)[0]
    assert h0.query_codes_offset == 0 and h0.query_exp_offset == 0
    assert (h0.partial_out_offset, h0.partial_lse_offset) == (h.partial_out_offset, h.partial_lse_offset)
    assert h0.workspace_bytes == h.query_codes_offset


def test_fp8_score_rejected_by_the_fused_variants():
    p = _qf8_params()
    st, plan = _plan(p, [0, 3, 8])
    assert st == m.MLA_OK
    h = m.read_plan(plan)[0]
    common = dict(params=p, plan_h=plan, workspace_d=FAKE, workspace_bytes=h.workspace_bytes,
                  q_nope_d=FAKE, q_nope_stride_n=128 * 512, q_nope_stride_h=512, q_rope_d=FAKE,
                  q_rope_stride_n=128 * 64, q_rope_stride_h=64, kv_cache_d=FAKE, kv_scale=0.5,
                  kv_indices_d=FAKE, sm_scale=0.1, out_d=FAKE, lse_d=None, stream=0)
    assert m.mla_decode_append(**common, c_new_d=FAKE, c_new_stride=576, k_pe_new_d=FAKE + 1024,
                               k_pe_new_stride=576) == m.MLA_ERR_UNSUPPORTED
    assert m.mla_decode_suffix_merge(**common, kv_lens_d=None, prefix_out_d=FAKE,
                                     prefix_lse_d=FAKE) == m.MLA_ERR_UNSUPPORTED
    # A plan built without the flag does not serve a call with it, nor the reverse.
    plain = m.make_params(128, 64, kv_dtype=m.MLA_DTYPE_FP8_E4M3FN, num_cus=256)
    assert m.mla_decode(**{**common, "params": plain}, kv_lens_d=None) == m.MLA_ERR_PLAN_MISMATCH


def test_noalloc_rejects_plans_beyond_its_scratch():
    """mla_decode_noalloc checks the plan's workspace needs against its fixed
    64 MiB scratch before touching the device (so this runs on the CPU)."""
    p = B.make_params(128, 64, num_cus=2048)
    lens = np.full(16, 200_000, np.int64)
    npages = (lens + 63) // 64
    indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    last = (lens - 64 * (npages - 1)).astype(np.int32)
    pb, wb = B.mla_decode_workspace_size(p, 16, 16)
    plan = np.zeros(pb, np.uint8)
    assert B.mla_decode_plan(p, 16, None, indptr, last, plan, pb) == B.MLA_OK
    h = B.read_plan(plan)[0]
    assert h.workspace_bytes > 64 << 20
    st = B.mla_decode_noalloc(p, plan, 16, 0, 0, 16, 0, 0, 16, 1.0, 16, None, 0.07, 16, None)
    assert st == B.MLA_ERR_WORKSPACE_TOO_SMALL
    bad = plan.copy()
    bad[:4] = 0  # not a plan
    st = B.mla_decode_noalloc(p, bad, 16, 0, 0, 16, 0, 0, 16, 1.0, 16, None, 0.07, 16, None)
    assert st == B.MLA_ERR_INVALID_ARG
