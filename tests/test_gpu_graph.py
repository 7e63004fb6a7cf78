"""A decode step (attention + split merge, plan made once beforehand) captured into a HIP graph and replayed:
the library launches kernels only -- no allocation, no memset, no host synchronisation -- so the step can be
captured.  Each replay runs on new query contents written in place between replays, with eager work and a
synchronisation in between, and must give the eager call's bits."""
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


@pytest.mark.parametrize("nwg", [0, 7])
def test_captured_step_replays_match_eager(torch, M, nwg):
    wl = W.make_workload("graph", batch=5, num_heads=32, seqlens=[70, 1300, 2, 640, 3000], s_q=2, causal=True,
                         seed=21)
    dev = torch.device("cuda")
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
    kv = torch.from_numpy(wl.cache.view(np.int16)).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seqlens).to(dev)
    mk = lambda: M.MlaDecode(batch=wl.batch, seqlen_q=wl.s_q, num_heads=wl.num_heads, num_pages=wl.num_pages,
                             max_blocks_per_seq=wl.block_table.shape[1], causal=True,
                             softmax_scale=float(wl.softmax_scale), num_workgroups=nwg)
    cap, ref = mk(), mk()
    cap.plan(sl)
    ref.plan(sl)
    torch.cuda.synchronize()
    _say(f"capture (nwg={nwg})")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cap.decode(q, kv, bt, sl)             # warm-up on the capture stream
        cap.combine()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cap.decode(q, kv, bt, sl)
        cap.combine()
    rng = np.random.default_rng(5)
    for rep in range(4):
        new_q = W.f32_to_bf16_bits(rng.standard_normal(wl.q.shape, dtype=np.float32))
        q.copy_(torch.from_numpy(new_q.view(np.int16)).to(dev))
        ref.decode(q, kv, bt, sl)             # eager work between replays
        ref.combine()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"replay {rep}")
        assert torch.equal(cap.out.view(torch.int16), ref.out.view(torch.int16)), f"replay {rep}: output"
        assert torch.equal(cap.lse.view(torch.int32), ref.lse.view(torch.int32)), f"replay {rep}: lse"
    assert cap.flags() == 0
