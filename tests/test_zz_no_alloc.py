"""The no-allocation decode step (mla_decode_noalloc) against the workspace path (mla_get_workspace +
mla_decode_fwd + mla_splitkv_combine) through the C ABI (MI355X only).

Both run the same kernels on the same plan, so the outputs must agree bit for bit (stronger than the tolerance
bar).  Two calls in a row, the second smaller than the first, so the fixed scratch is reused with stale contents
from a bigger step; each call is also checked against the fp64 oracle.  A step whose workspace exceeds the
scratch is rejected before anything runs.  Collected last (test_zz_*): it must pass both alone in a fresh process
and after the other GPU tests."""
import ctypes

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _say, check, oracle, run_gpu, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("no GPU visible")
    return t


@pytest.fixture(scope="module")
def M():
    import mla_latent_kv_fwd_amd as m
    m.load_library()
    return m


def _noalloc(torch, M, wl, tensors):
    q, kv, ks, bt, sl = tensors
    p = M.make_params(batch=wl.batch, seqlen_q=wl.s_q, num_heads=wl.num_heads, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], causal=wl.causal,
                      kv_dtype=M.MLA_KV_FP8_E4M3FN if wl.kv_dtype == "fp8_e4m3fn" else M.MLA_KV_BF16,
                      softmax_scale=float(wl.softmax_scale))
    out = torch.full((wl.batch, wl.s_q, wl.num_heads, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((wl.batch, wl.s_q, wl.num_heads), 7.0, dtype=torch.float32, device="cuda")
    M.mla_decode_noalloc(p, q.data_ptr(), kv.data_ptr(), 0 if ks is None else ks.data_ptr(), bt.data_ptr(),
                         sl.data_ptr(), out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


@pytest.mark.parametrize("order", ["bf16", "fp8"])
def test_noalloc_matches_workspace_path_twice(torch, M, order):
    big = W.make_workload("na-big", batch=9, num_heads=128, seqlens=[5000, 64, 700, 3000, 2, 129, 4096, 3, 900],
                          s_q=2, causal=True, seed=71, spare_pages=3,
                          kv_dtype="fp8_e4m3fn" if order == "fp8" else "bf16")
    small = W.make_workload("na-small", batch=3, num_heads=32, seqlens=[300, 77, 1500], seed=72, spare_pages=2,
                            kv_dtype="fp8_e4m3fn" if order == "fp8" else "bf16")
    for wl in (big, small):
        _say(f"no-alloc {order} {wl.name}")
        t = to_gpu(torch, wl)
        o_ref, l_ref, _ = run_gpu(torch, M, wl, tensors=t)
        o, l = _noalloc(torch, M, wl, t)
        assert np.array_equal(o, o_ref), f"{wl.name}: output bits differ from the workspace path"
        assert np.array_equal(l.view(np.uint32), l_ref.view(np.uint32)), f"{wl.name}: lse bits differ"
        ref_o, ref_l = oracle(wl)
        check(o, l, ref_o, ref_l, f"no-alloc {order} {wl.name}")


def test_noalloc_rejects_a_step_beyond_the_scratch(torch, M):
    wl = W.make_workload("na-huge", batch=64, num_heads=128, seqlens=[4096] * 64, seed=73)
    t = to_gpu(torch, wl)
    q, kv, _, bt, sl = t
    p = M.make_params(batch=64, seqlen_q=1, num_heads=128, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], num_workgroups=4096)
    assert M.mla_get_workspace(p) > M.MLA_NOALLOC_SCRATCH_BYTES
    out = torch.empty((64, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((64, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MlaError) as e:
        M.mla_decode_noalloc(p, q.data_ptr(), kv.data_ptr(), 0, bt.data_ptr(), sl.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert e.value.status == M.MLA_ERR_SCRATCH_TOO_SMALL
