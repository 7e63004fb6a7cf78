"""The Python binding's argument checks (CPU only): every tensor mla_decode_fwd reads is checked against the
parameters before a device pointer is passed on, so a wrongly typed or sized tensor raises instead of being read
out of bounds by the kernel."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import mla_latent_kv_fwd_amd as M  # noqa: E402


def _params(fp8=False, **kw):
    d = dict(batch=2, seqlen_q=1, num_heads=16, num_pages=5, max_blocks_per_seq=3,
             kv_dtype=M.MLA_KV_FP8_E4M3FN if fp8 else M.MLA_KV_BF16)
    d.update(kw)
    return M.make_params(**d)


def _tensors(p, fp8=False):
    q = torch.zeros((p.batch, p.seqlen_q, p.num_heads, 576), dtype=torch.bfloat16)
    kv = torch.zeros((p.num_pages, 64, 576), dtype=torch.uint8 if fp8 else torch.bfloat16)
    ks = torch.ones((p.num_pages, 64), dtype=torch.float32) if fp8 else None
    bt = torch.zeros((p.batch, p.max_blocks_per_seq), dtype=torch.int32)
    sl = torch.ones((p.batch,), dtype=torch.int32)
    return q, kv, bt, sl, ks


@pytest.mark.parametrize("fp8", [False, True])
def test_matching_tensors_pass(fp8):
    p = _params(fp8)
    q, kv, bt, sl, ks = _tensors(p, fp8)
    M.check_decode_inputs(p, "cpu", q, kv, bt, sl, ks)
    M.check_decode_inputs(p, "cpu", q.view(torch.int16), kv, bt, sl, ks)   # bf16 bits as int16 are accepted


@pytest.mark.parametrize("what", ["q_shape", "q_dtype", "q_noncontig", "kv_pages", "kv_width", "kv_dtype",
                                  "bt_int64", "bt_shape", "sl_int64", "sl_shape", "scale_given_for_bf16",
                                  "device"])
def test_bf16_mismatches_raise(what):
    p = _params()
    q, kv, bt, sl, ks = _tensors(p)
    if what == "q_shape":
        q = q[:, :, :8]
    elif what == "q_dtype":
        q = q.float()
    elif what == "q_noncontig":
        q = torch.zeros((p.batch, p.seqlen_q, 576, p.num_heads), dtype=torch.bfloat16).transpose(2, 3)
    elif what == "kv_pages":
        kv = kv[:4]
    elif what == "kv_width":
        kv = torch.zeros((p.num_pages, 64, 512), dtype=torch.bfloat16)
    elif what == "kv_dtype":
        kv = kv.float()
    elif what == "bt_int64":
        bt = bt.long()
    elif what == "bt_shape":
        bt = bt[:, :2].contiguous()
    elif what == "sl_int64":
        sl = sl.long()
    elif what == "sl_shape":
        sl = torch.ones((3,), dtype=torch.int32)
    elif what == "scale_given_for_bf16":
        ks = torch.ones((p.num_pages, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        M.check_decode_inputs(p, "meta" if what == "device" else "cpu", q, kv, bt, sl, ks)


@pytest.mark.parametrize("what", ["no_scale", "scale_f16", "scale_shape", "kv_16bit"])
def test_fp8_mismatches_raise(what):
    p = _params(fp8=True)
    q, kv, bt, sl, ks = _tensors(p, fp8=True)
    if what == "no_scale":
        ks = None
    elif what == "scale_f16":
        ks = ks.half()
    elif what == "scale_shape":
        ks = ks[:4]
    elif what == "kv_16bit":
        kv = torch.zeros((p.num_pages, 64, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        M.check_decode_inputs(p, "cpu", q, kv, bt, sl, ks)


def test_debug_flag_text_and_environment(monkeypatch):
    import mla_latent_kv_fwd_amd as M
    assert M.describe_flags(0) == "none"
    text = M.describe_flags(M.MLA_FLAG_SEQLEN_CLAMPED | M.MLA_FLAG_BAD_PLAN)
    assert "clamped" in text and "plan" in text and "block-table" not in text
    monkeypatch.setenv("MLA_DEBUG", "1")
    assert M.debug_from_env()
    monkeypatch.setenv("MLA_DEBUG", "0")
    assert not M.debug_from_env()
    monkeypatch.delenv("MLA_DEBUG")
    assert not M.debug_from_env()


def test_debug_checks_of_lengths_and_used_pages():
    """The debug mode's host-side checks (MlaDecode.check_device_values), run on CPU tensors."""
    import torch
    import mla_latent_kv_fwd_amd as M

    class Holder:
        params = M.make_params(batch=2, seqlen_q=1, num_heads=16, num_pages=4, max_blocks_per_seq=4)

    check = lambda bt, sl: M.MlaDecode.check_device_values(Holder(), torch.tensor(bt, dtype=torch.int32),
                                                           torch.tensor(sl, dtype=torch.int32))
    good = [[1, 2, -1, -1], [3, 0, -1, -1]]
    check(good, [100, 100])
    check([[1, 2, -1, -7], [3, 0, -1, -1]], [100, 100])   # an entry past a request's pages is not read
    with pytest.raises(M.MlaDeviceError) as e:
        check([[1, 2, -1, -1], [3, 9, -1, -1]], [100, 100])
    assert e.value.flags == M.MLA_FLAG_BAD_BLOCK and "block_table[1][1] = 9" in str(e.value)
    with pytest.raises(M.MlaDeviceError) as e:
        check(good, [100, 257])                             # beyond 4 pages of 64
    assert e.value.flags == M.MLA_FLAG_SEQLEN_CLAMPED
    with pytest.raises(M.MlaDeviceError):
        check(good, [0, 100])                               # below seqlen_q
