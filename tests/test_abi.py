"""The C ABI boundary, checked without a GPU: the library loads, exports every
function include/*.h declares, and rejects bad arguments with the documented
status codes before anything is enqueued."""
import ctypes
import glob
import os
import re

import pytest

import mla_latent_kv_fwd_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmla_decode.so is not built (python -m mla_latent_kv_fwd_amd.build)")
    return M.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(M.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_function(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (M.MLA_OK, M.MLA_ERR_INVALID_ARG, M.MLA_ERR_UNSUPPORTED, M.MLA_ERR_WORKSPACE_TOO_SMALL, M.MLA_ERR_HIP):
        assert lib.mla_status_string(st) not in (None, b"", b"unknown status")


def _params(**kw):
    base = dict(batch=4, seqlen_q=1, num_heads=128, num_pages=64, max_blocks_per_seq=16, num_workgroups=32)
    base.update(kw)
    return M.make_params(**base)


def _status(call):
    with pytest.raises(M.MlaError) as e:
        call()
    return e.value.status


def test_size_query_needs_no_device(lib):
    small = M.mla_get_workspace(_params())
    big = M.mla_get_workspace(_params(num_workgroups=64))
    assert 0 < small < big                       # partial buffers grow with the stretches
    assert M.mla_get_workspace(_params(seqlen_q=2)) > small   # and with the row blocks


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, M.MLA_ERR_INVALID_ARG),
    ("seqlen_q", 0, M.MLA_ERR_INVALID_ARG),
    ("num_heads", 0, M.MLA_ERR_INVALID_ARG),
    ("num_pages", 0, M.MLA_ERR_INVALID_ARG),
    ("max_blocks_per_seq", 0, M.MLA_ERR_INVALID_ARG),
    ("num_workgroups", -1, M.MLA_ERR_INVALID_ARG),
    ("softmax_scale", 0.0, M.MLA_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), M.MLA_ERR_INVALID_ARG),
    ("kv_dtype", 7, M.MLA_ERR_INVALID_ARG),
    ("head_dim_qk", 192, M.MLA_ERR_UNSUPPORTED),
    ("head_dim_v", 128, M.MLA_ERR_UNSUPPORTED),
    ("page_size", 16, M.MLA_ERR_UNSUPPORTED),
    ("num_heads", 129, M.MLA_ERR_UNSUPPORTED),
    ("seqlen_q", 9, M.MLA_ERR_UNSUPPORTED),
    ("fp8_path", 2, M.MLA_ERR_INVALID_ARG),
    ("fp8_path", -1, M.MLA_ERR_INVALID_ARG),
    ("fp8_path", 1, M.MLA_ERR_INVALID_ARG),      # the E4M3 route needs an FP8 cache
])
def test_bad_params_are_rejected(lib, field, value, status):
    p = _params()
    setattr(p, field, value)
    assert _status(lambda: M.mla_get_workspace(p)) == status
    assert _status(lambda: M.mla_decode_fwd(p, 16, 16, 0, 16, 16, 256, 1 << 30, 16, 16)) == status
    assert _status(lambda: M.mla_splitkv_combine(p, 256, 1 << 30, 16, 16)) == status


def test_null_and_misaligned_pointers_are_rejected(lib):
    p = _params()
    n = M.mla_get_workspace(p)
    ok = dict(q_ptr=16, kv_ptr=16, kv_scale_ptr=0, block_table_ptr=16, seqlens_ptr=16, workspace_ptr=256,
              workspace_bytes=n, out_ptr=16, lse_ptr=16)
    for name in ("q_ptr", "kv_ptr", "block_table_ptr", "seqlens_ptr", "workspace_ptr", "out_ptr", "lse_ptr"):
        args = dict(ok, **{name: 0})
        assert _status(lambda: M.mla_decode_fwd(p, **args)) == M.MLA_ERR_INVALID_ARG, name
    assert _status(lambda: M.mla_decode_fwd(p, **dict(ok, workspace_ptr=260))) == M.MLA_ERR_INVALID_ARG
    assert _status(lambda: M.mla_decode_fwd(p, **dict(ok, q_ptr=18))) == M.MLA_ERR_INVALID_ARG
    # a scale pointer with a bf16 cache is a contract violation
    assert _status(lambda: M.mla_decode_fwd(p, **dict(ok, kv_scale_ptr=64))) == M.MLA_ERR_INVALID_ARG
    # plan: no seqlens, misaligned or undersized workspace
    assert _status(lambda: M.mla_get_workspace(p, 0, 256, n)) == M.MLA_ERR_INVALID_ARG
    assert _status(lambda: M.mla_get_workspace(p, 16, 272, n)) == M.MLA_ERR_INVALID_ARG
    assert _status(lambda: M.mla_get_workspace(p, 16, 256, n - 1)) == M.MLA_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: M.mla_decode_fwd(p, **dict(ok, workspace_bytes=n - 1))) == M.MLA_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: M.mla_splitkv_combine(p, 256, n - 1, 16, 16)) == M.MLA_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: M.mla_workspace_flags(0)) == M.MLA_ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        M._lib, saved = None, M._lib
        try:
            M.load_library(str(tmp_path / "nope.so"))
        finally:
            M._lib = saved


def _proj_params(**kw):
    base = dict(tokens=64, num_heads=128)
    base.update(kw)
    return M.make_proj_params(**base)


@pytest.mark.parametrize("field,value,status", [
    ("tokens", 0, M.MLA_ERR_INVALID_ARG),
    ("tokens", 65537, M.MLA_ERR_INVALID_ARG),
    ("num_heads", 0, M.MLA_ERR_INVALID_ARG),
    ("num_heads", 129, M.MLA_ERR_UNSUPPORTED),
    ("d_nope", 64, M.MLA_ERR_UNSUPPORTED),
    ("d_rope", 32, M.MLA_ERR_UNSUPPORTED),
    ("d_latent", 256, M.MLA_ERR_UNSUPPORTED),
    ("d_v", 64, M.MLA_ERR_UNSUPPORTED),
])
def test_bad_projection_params_are_rejected(lib, field, value, status):
    p = _proj_params()
    setattr(p, field, value)
    assert _status(lambda: M.mla_absorb_q(p, 16, 16, 16, 16)) == status
    assert _status(lambda: M.mla_project_out(p, 16, 16, 16)) == status


def test_projection_pointers_are_checked(lib):
    p = _proj_params()
    for args in ((0, 16, 16, 16), (16, 0, 16, 16), (16, 16, 0, 16), (16, 16, 16, 0), (24, 16, 16, 16),
                 (16, 16, 16, 8)):
        assert _status(lambda: M.mla_absorb_q(p, *args)) == M.MLA_ERR_INVALID_ARG, args
    for args in ((0, 16, 16), (16, 0, 16), (16, 16, 0), (16, 32, 40)):
        assert _status(lambda: M.mla_project_out(p, *args)) == M.MLA_ERR_INVALID_ARG, args


def _pf_params(**kw):
    base = dict(num_heads=128, num_new=64, seqlen=1000, num_pages=20, max_blocks=16, chunk_tokens=256)
    base.update(kw)
    return M.make_prefill_params(**base)


@pytest.mark.parametrize("field,value,status", [
    ("num_heads", 0, M.MLA_ERR_INVALID_ARG),
    ("num_heads", 129, M.MLA_ERR_UNSUPPORTED),
    ("num_new", 0, M.MLA_ERR_INVALID_ARG),
    ("num_new", 65537, M.MLA_ERR_INVALID_ARG),
    ("seqlen", 63, M.MLA_ERR_INVALID_ARG),          # fewer tokens than new tokens
    ("seqlen", 16 * 64 + 1, M.MLA_ERR_INVALID_ARG),  # more than the block-table row holds
    ("num_pages", 0, M.MLA_ERR_INVALID_ARG),
    ("chunk_tokens", 0, M.MLA_ERR_INVALID_ARG),
    ("chunk_tokens", 100, M.MLA_ERR_INVALID_ARG),
    ("chunk_tokens", 65600, M.MLA_ERR_INVALID_ARG),
    ("softmax_scale", 0.0, M.MLA_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), M.MLA_ERR_INVALID_ARG),
    ("d_nope", 64, M.MLA_ERR_UNSUPPORTED),
    ("d_latent", 256, M.MLA_ERR_UNSUPPORTED),
])
def test_bad_prefill_params_are_rejected(lib, field, value, status):
    p = _pf_params()
    setattr(p, field, value)
    assert _status(lambda: M.mla_prefill_workspace_size(p)) == status
    assert _status(lambda: M.mla_expand_kv(p, 16, 16, 0, 64, 16, 16, 16, 16)) == status
    assert _status(lambda: M.mla_prefill_attention(p, 16, 16, 16, 0, 64, 16, 16)) == status
    assert _status(lambda: M.mla_chunked_prefill(p, 16, 16, 16, 16, 16, 256, 1 << 40, 16, 16)) == status


def test_prefill_ranges_and_pointers_are_checked(lib):
    p = _pf_params()
    for t0, ntok in ((-1, 10), (0, 0), (990, 11), (0, 1001)):
        assert _status(lambda: M.mla_expand_kv(p, 16, 16, t0, ntok, 16, 16, 16, 16)) == M.MLA_ERR_INVALID_ARG
        assert _status(lambda: M.mla_prefill_attention(p, 16, 16, 16, t0, ntok, 16, 16)) == M.MLA_ERR_INVALID_ARG
    for args in ((0, 16, 16, 16, 16, 16), (24, 16, 16, 16, 16, 16), (16, 16, 16, 16, 16, 8)):
        cache, bt, wuk, wuv, k, vt = args
        assert _status(lambda: M.mla_expand_kv(p, cache, bt, 0, 64, wuk, wuv, k, vt)) == M.MLA_ERR_INVALID_ARG
    assert _status(lambda: M.mla_prefill_attention(p, 16, 16, 16, 0, 64, 16, 18)) == M.MLA_ERR_INVALID_ARG
    # workspace: misaligned, then too small
    assert _status(lambda: M.mla_chunked_prefill(p, 16, 16, 16, 16, 16, 128, 1 << 40, 16, 16)) == \
        M.MLA_ERR_INVALID_ARG
    need = M.mla_prefill_workspace_size(p)
    assert _status(lambda: M.mla_chunked_prefill(p, 16, 16, 16, 16, 16, 256, need - 1, 16, 16)) == \
        M.MLA_ERR_WORKSPACE_TOO_SMALL


def test_prefill_workspace_covers_every_chunk(lib):
    """One K and V^T chunk (H x Tc x (192 + 128) bf16) plus fp32 partials and LSEs of all chunks."""
    p = _pf_params(num_heads=8, num_new=10, seqlen=1000, chunk_tokens=256)
    need = M.mla_prefill_workspace_size(p)
    chunks = 4
    assert need >= 8 * 256 * 320 * 2 + chunks * 10 * 8 * (128 + 1) * 4
    assert need % 256 == 0


@pytest.mark.parametrize("rows,parts", [(0, 1), (1, 0), (1, 4097), (1 << 24 | 1, 2)])
def test_bad_merge_sizes_are_rejected(lib, rows, parts):
    assert _status(lambda: M.mla_lse_merge(rows, parts, 16, 16, 16, 16)) == M.MLA_ERR_INVALID_ARG


def test_merge_pointers_are_checked(lib):
    for args in ((0, 16, 16, 16), (8, 16, 16, 16), (16, 18, 16, 16), (16, 16, 8, 16), (16, 16, 16, 2)):
        assert _status(lambda: M.mla_lse_merge(4, 2, *args)) == M.MLA_ERR_INVALID_ARG
