"""The split plan's invariants, read back from the workspace after the plan kernel
runs on the GPU (white-box: the workspace layout is the library's internal one).

For random length mixes and stretch counts: the stretches partition the
concatenated pages in order; each request's page range matches its clamped
length; the stretches holding a request are counted by nsplit and numbered
0..nsplit-1 by (ne_prefix - ne_lo); split requests get disjoint partial-slot
ranges inside the reserved 2 * stretches; stretch costs are balanced, and
equal requests split into equal pieces."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

PAGE = 64
COST_PER_REQUEST = 3


def _align(x):
    return (x + 255) & ~255


def _layout(batch, nwg):
    off = _align(64)                     # header
    wg = off
    off = _align(off + 32 * nwg)
    req = off
    return wg, req


@pytest.fixture(scope="module")
def env():
    import torch
    import mla_latent_kv_fwd_amd as M
    M.load_library()
    return torch, M


def _plan(torch, M, seqlens, nwg, max_blocks, s_q=1):
    B = len(seqlens)
    p = M.make_params(batch=B, seqlen_q=s_q, num_heads=128, num_pages=max(1, B * max_blocks),
                      max_blocks_per_seq=max_blocks, num_workgroups=nwg)
    nbytes = M.mla_get_workspace(p)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    M.mla_get_workspace(p, sl.data_ptr(), ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    nwg_eff = int(raw[16:20].view(np.int32)[0])
    wg_off, req_off = _layout(B, nwg_eff)
    wg = raw[wg_off:wg_off + 32 * nwg_eff].view(np.int32).reshape(nwg_eff, 8)
    req = raw[req_off:req_off + 32 * B].view(np.int32).reshape(B, 8)
    hdr = raw[:64].view(np.int32)
    return hdr, wg, req, nwg_eff


@pytest.mark.parametrize("seed", range(10))
def test_plan_invariants(env, seed):
    torch, M = env
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 3, 64, 128, 1000]))
    max_blocks = int(rng.choice([4, 64, 512]))
    seqlens = rng.integers(1, max_blocks * PAGE + 1, B)
    if seed % 2:
        seqlens[rng.integers(0, B, max(1, B // 10))] = 1     # sprinkle one-token requests
    if seed >= 6:
        seqlens[:] = seqlens[0]                              # equal lengths: the even split
    nwg = int(rng.choice([1, 2, 7, 64, 256, 1000]))
    hdr, wg, req, nwg_eff = _plan(torch, M, seqlens, nwg, max_blocks)

    npages = (np.minimum(seqlens, max_blocks * PAGE) + PAGE - 1) // PAGE
    first = np.concatenate([[0], np.cumsum(npages)[:-1]])
    total = int(npages.sum())
    assert hdr[7] == total                                   # header.total_pages
    assert np.array_equal(req[:, 0], first) and np.array_equal(req[:, 1], npages)
    assert np.array_equal(req[:, 5], seqlens)

    # stretches partition [0, total) in order
    assert wg[0, 0] == 0 and wg[-1, 1] == total
    assert np.array_equal(wg[1:, 0], wg[:-1, 1])
    nonempty = wg[:, 1] > wg[:, 0]
    assert np.array_equal(wg[:, 3], np.concatenate([[0], np.cumsum(nonempty)[:-1]]))

    slots = []
    for b in range(B):
        holders = [s for s in range(nwg_eff) if nonempty[s] and wg[s, 0] < first[b] + npages[b]
                   and wg[s, 1] > first[b]]
        assert req[b, 2] == len(holders), (b, holders)
        assert [wg[s, 3] - req[b, 4] for s in holders] == list(range(len(holders)))
        if req[b, 2] > 1:
            slots.append((req[b, 3], req[b, 3] + req[b, 2]))
    for s in range(nwg_eff):
        if nonempty[s]:
            b = wg[s, 2]
            assert first[b] <= wg[s, 0] < first[b] + npages[b]
            assert wg[s, 4] == wg[s, 0] - first[b]               # request-local first page
    slots.sort()
    for (a0, a1), (b0, _) in zip(slots, slots[1:]):
        assert a1 <= b0
    if slots:
        assert slots[0][0] >= 0 and slots[-1][1] <= 2 * nwg_eff
    assert hdr[8] == sum(e - s for s, e in slots)           # header.used_slots

    # balance: no stretch costs more than the fair share plus one page and one request's
    # fixed cost.  Lengths that differ: the fixed cost is charged where a request starts;
    # equal lengths: it is spread over the request's pages (every piece of a split request
    # pays its own), so a page weighs (np + c) / np and each cut lies within half a page
    # of its exact cost position
    uniform = len(set(npages.tolist())) == 1
    cost_of = np.zeros(nwg_eff)
    for s in range(nwg_eff):
        lo, hi = wg[s, 0], wg[s, 1]
        for b in range(B):
            ov = min(hi, first[b] + npages[b]) - max(lo, first[b])
            if ov > 0:
                if uniform:
                    cost_of[s] += ov * (npages[b] + COST_PER_REQUEST) / npages[b]
                else:
                    cost_of[s] += ov + (COST_PER_REQUEST if lo <= first[b] else 0)
    fair = (total + COST_PER_REQUEST * int((npages > 0).sum())) / nwg_eff
    assert cost_of.max() <= fair + 1 + COST_PER_REQUEST + 1e-9


def test_plan_flags_out_of_range_lengths(env):
    torch, M = env
    hdr, wg, req, _ = _plan(torch, M, [0, 10_000, 5], nwg=4, max_blocks=4)
    assert hdr[1] & M.MLA_FLAG_SEQLEN_CLAMPED
    assert list(req[:, 5]) == [0, 256, 5] and list(req[:, 1]) == [0, 4, 1]


def test_plan_equal_requests_split_evenly(env):
    """64 requests of 4,096 tokens over 256 stretches: 16 pages each (every piece pays
    its own fixed cost, so the pieces of equal requests are equal)."""
    torch, M = env
    hdr, wg, req, nwg_eff = _plan(torch, M, [4096] * 64, nwg=256, max_blocks=64)
    assert nwg_eff == 256
    assert np.all(wg[:, 1] - wg[:, 0] == 16)
    assert np.all(req[:, 2] == 4)
