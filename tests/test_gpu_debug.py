"""MlaDecode's debug mode (MLA_DEBUG=1 or debug=True) on the GPU: synchronous checks of the device-side values
before the launch, and a raise on any workspace flag after decode + combine.  Bad values are caught on the host
before any kernel runs; the flag path is driven by a workspace that holds no plan, which the kernels turn into
the defined empty result without reading a plan entry."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


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


def _setup(torch, M, wl, debug):
    dev = torch.device("cuda")
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
    kv = torch.from_numpy(wl.cache.view(np.int16)).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seqlens).to(dev)
    dec = M.MlaDecode(batch=wl.batch, seqlen_q=wl.s_q, num_heads=wl.num_heads, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], softmax_scale=float(wl.softmax_scale), debug=debug)
    return dec, q, kv, bt, sl


def test_debug_mode_matches_the_plain_call(torch, M):
    wl = W.make_workload("dbg_ok", batch=3, num_heads=16, seqlens=[100, 1, 700], seed=11)
    _say("debug mode, valid inputs")
    plain, q, kv, bt, sl = _setup(torch, M, wl, debug=False)
    o0, l0 = plain(q, kv, bt, sl)
    dbg = _setup(torch, M, wl, debug=True)[0]
    o1, l1 = dbg(q, kv, bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))


def test_debug_mode_rejects_bad_lengths_and_pages_before_launch(torch, M):
    wl = W.make_workload("dbg_bad", batch=2, num_heads=16, seqlens=[100, 100], seed=12, max_blocks=4)
    dec, q, kv, bt, sl = _setup(torch, M, wl, debug=True)
    _say("debug mode, length past the block table")
    long_sl = sl.clone()
    long_sl[1] = wl.block_table.shape[1] * 64 + 1
    with pytest.raises(M.MlaDeviceError) as e:
        dec(q, kv, bt, long_sl)
    assert e.value.flags == M.MLA_FLAG_SEQLEN_CLAMPED and "seqlens[1]" in str(e.value)
    _say("debug mode, block-table entry outside the cache")
    bad_bt = bt.clone()
    bad_bt[1, 1] = wl.num_pages + 5
    with pytest.raises(M.MlaDeviceError) as e:
        dec(q, kv, bad_bt, sl)
    assert e.value.flags == M.MLA_FLAG_BAD_BLOCK and "block_table[1][1]" in str(e.value)
    # An entry past the request's last page is not used, so it is not an error.
    unused = bt.clone()
    unused[0, -1] = -7
    dec(q, kv, unused, sl)
    torch.cuda.synchronize()


def test_debug_mode_raises_on_a_kernel_flag(torch, M):
    wl = W.make_workload("dbg_flag", batch=2, num_heads=16, seqlens=[300, 77], seed=13)
    dec, q, kv, bt, sl = _setup(torch, M, wl, debug=True)
    _say("debug mode, workspace without a plan")
    dec.workspace.zero_()
    with pytest.raises(M.MlaDeviceError) as e:
        dec(q, kv, bt, sl, plan=False)
    assert e.value.flags & M.MLA_FLAG_BAD_PLAN
    dec(q, kv, bt, sl)                       # planned: no flag
    torch.cuda.synchronize()
