"""HIP path vs the fp64 oracle, element by element, through the C ABI (MI355X only).

Tolerances (bf16 inputs, fp32 accumulation): output max-abs <= 2e-2 and relative
L2 <= 5e-3 over the whole tensor; LSE max-abs <= 1e-3.  Block-table indexing is
checked bit-exactly (a permuted physical layout of the same logical cache gives
identical bits), and a one-token request must reproduce its latent's bits.
The full-size configurations (headline, ragged batch, two new tokens; the FP8
cache in test_gpu_fp8.py) are compared on every row of the output, with the
worst row reported.
"""
import math
import os
import sys

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


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


def to_gpu(torch, wl):
    dev = torch.device("cuda")
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
    if wl.cache.dtype == np.uint16:
        kv = torch.from_numpy(wl.cache.view(np.int16)).to(dev)
    else:
        kv = torch.from_numpy(wl.cache).to(dev)
    ks = None if wl.kv_scale is None else torch.from_numpy(wl.kv_scale).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seqlens).to(dev)
    return q, kv, ks, bt, sl


def run_gpu(torch, M, wl, num_workgroups=0, tensors=None, fp8_path=0):
    q, kv, ks, bt, sl = tensors if tensors is not None else to_gpu(torch, wl)
    dec = M.MlaDecode(batch=wl.batch, seqlen_q=wl.s_q, num_heads=wl.num_heads, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], causal=wl.causal,
                      kv_dtype=M.MLA_KV_FP8_E4M3FN if wl.kv_dtype == "fp8_e4m3fn" else M.MLA_KV_BF16,
                      softmax_scale=float(wl.softmax_scale), num_workgroups=num_workgroups, fp8_path=fp8_path)
    out, lse = dec(q, kv, bt, sl, ks)
    torch.cuda.synchronize()
    flags = dec.flags()
    out_np = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out_np, lse.cpu().numpy(), flags


def oracle(wl, rows=None):
    return O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=wl.causal,
                    kv_scale=wl.kv_scale, rows=rows)


def check(out_bits, lse, ref_out, ref_lse, what, max_abs=OUT_MAX_ABS):
    got = W.bf16_bits_to_f32(out_bits).astype(np.float64).reshape(ref_out.shape)
    lse = np.asarray(lse, np.float64).reshape(ref_lse.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref_out)
    rel = np.linalg.norm(got - ref_out) / max(np.linalg.norm(ref_out), 1e-30)
    lerr = np.abs(lse - ref_lse)
    d2 = (got - ref_out).reshape(-1, got.shape[-1])
    r2 = ref_out.reshape(-1, got.shape[-1])
    row_rel = np.linalg.norm(d2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
    _say(f"{what}: out max-abs {err.max():.3e} rel-L2 {rel:.3e} (worst row {int(row_rel.argmax())}: "
         f"{row_rel.max():.3e})  lse max-abs {lerr.max():.3e}  [{d2.shape[0]} rows]")
    assert err.max() <= max_abs, f"{what}: out max-abs {err.max()}"
    assert rel <= OUT_REL_L2, f"{what}: out rel-L2 {rel}"
    assert lerr.max() <= LSE_MAX_ABS, f"{what}: lse max-abs {lerr.max()}"


# ------------------------------------------------------------------ small, full comparison
def test_tiny_config(torch, M):
    wl = W.make_config("tiny_b1_h16_l256")
    _say("tiny_b1_h16_l256")
    out, lse, flags = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, "tiny")
    assert flags == 0


def test_ragged_triple_from_the_guide(torch, M):
    """Three requests of 450, 18,200 and 3,100 tokens (the FlashMLA guide's ragged-batching example)."""
    wl = W.make_workload("ragged3", batch=3, num_heads=128, seqlens=[450, 18200, 3100], seed=31, spare_pages=4)
    _say("ragged triple 450/18200/3100")
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, "ragged3")


@pytest.mark.parametrize("nwg", [1, 2, 3, 7, 16, 64, 256])
def test_split_invariance(torch, M, nwg):
    """Any number of stretches (1 = nothing split, many = every request split) matches the oracle."""
    wl = W.make_workload("splits", batch=5, num_heads=128, seqlens=[64, 1, 700, 2049, 130], seed=7, spare_pages=3)
    _say(f"split invariance nwg={nwg}")
    out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"nwg={nwg}")


@pytest.mark.parametrize("L", [1, 2, 3, 4, 31, 32, 33, 63, 64, 65, 127, 129])
def test_short_lengths(torch, M, L):
    wl = W.make_workload(f"short{L}", batch=2, num_heads=128, seqlens=[L, L + 1], seed=100 + L, spare_pages=2)
    _say(f"short lengths L={L}")
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"L={L}")


JUMP_SEQLENS = [1600, 900, 1100, 2000, 1800]
JUMP_SPANS = [[(1200, 3, 1)],                              # mid-request, inside a page
              [(896, 3, 1)],                               # in the ragged last page
              [(0, 3, 1)],                                 # first chunk: later keys sit far below the maximum
              [(600, 1, 1), (1300, 1, 1), (1999, 1, 1)],   # one jump, then more keys at the same level
              [(1000, 3, 1), (1700, 1, 2)]]                # two jumps: two rescales of the running sums


@pytest.mark.parametrize("nwg", [0, 1, 7])
def test_score_jump_forces_rescale(torch, M, nwg):
    """Scores that rise by ~9.4 (log2 units) partway through a request make the
    running maximum rescale the accumulated output and normaliser, while the
    earlier keys still carry ~40% of the softmax mass."""
    wl = W.make_score_jump_workload("jump", seqlens=JUMP_SEQLENS, jumps=JUMP_SPANS, seed=41)
    _say(f"score jumps nwg={nwg}")
    out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"jump nwg={nwg}")


def test_one_token_copies_latent_bits(torch, M):
    """With one visible token p = 1 exactly, so the bf16 output must equal the cached latent bit for bit."""
    wl = W.make_workload("one", batch=4, num_heads=128, seqlens=[1, 1, 1, 1], seed=3)
    out, lse, _ = run_gpu(torch, M, wl)
    for b in range(4):
        lat = wl.cache[wl.block_table[b, 0], 0, :512]
        assert np.array_equal(out[b, 0], np.broadcast_to(lat, (128, 512)))
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, "one token")


@pytest.mark.parametrize("H,s_q", [(16, 1), (32, 1), (64, 1), (128, 2), (64, 2), (16, 2), (1, 1), (20, 3), (3, 8),
                                 (128, 8)])
def test_head_counts_and_new_tokens(torch, M, H, s_q):
    wl = W.make_workload(f"h{H}s{s_q}", batch=3, num_heads=H, seqlens=[300, 77, 1500], s_q=s_q, causal=s_q > 1,
                         seed=H + s_q, spare_pages=2)
    _say(f"H={H} s_q={s_q}")
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"H={H} s_q={s_q}")


def test_causal_last_token_only_in_last_row(torch, M):
    """s_q = 2 with a split boundary right before the last page: row 0 sees none of the last stretch."""
    wl = W.make_workload("causal-edge", batch=1, num_heads=128, seqlens=[129], s_q=2, causal=True, seed=5)
    for nwg in (1, 3, 4):
        out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg)
        ref_o, ref_l = oracle(wl)
        check(out, lse, ref_o, ref_l, f"causal edge nwg={nwg}")


# ------------------------------------------------------------------ bit-exact indexing, poison
def test_block_table_permutation_is_bit_exact(torch, M):
    wl = W.make_workload("perm", batch=4, num_heads=128, seqlens=[1000, 64, 333, 2000], seed=12, spare_pages=5)
    out1, lse1, _ = run_gpu(torch, M, wl)
    # rebuild the same logical cache under another physical permutation
    rng = np.random.default_rng(99)
    P = wl.num_pages
    perm = rng.permutation(P).astype(np.int32)
    cache2 = np.empty_like(wl.cache)
    cache2[perm] = wl.cache
    bt2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    wl2 = W.Workload(name="perm2", q=wl.q, cache=cache2, kv_scale=None, block_table=bt2, seqlens=wl.seqlens,
                     s_q=wl.s_q, num_heads=wl.num_heads, causal=wl.causal)
    out2, lse2, _ = run_gpu(torch, M, wl2)
    assert np.array_equal(out1, out2)
    assert np.array_equal(lse1.view(np.uint32), lse2.view(np.uint32))


def test_nan_poison_outside_lengths_is_ignored(torch, M):
    wl = W.make_workload("poison", batch=6, num_heads=128, seqlens=[1, 63, 65, 127, 500, 4097], seed=17,
                         spare_pages=8, poison=True)
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, "poison")


# ------------------------------------------------------------------ contract violations (host-forced)
def test_bad_block_entry_sets_flag_without_fault(torch, M):
    wl = W.make_workload("badbt", batch=2, num_heads=16, seqlens=[100, 100], seed=2)
    bt = wl.block_table.copy()
    bt[1, 1] = wl.num_pages + 5          # outside the cache: must not be dereferenced
    wl2 = W.Workload(name="badbt2", q=wl.q, cache=wl.cache, kv_scale=None, block_table=bt, seqlens=wl.seqlens,
                     s_q=1, num_heads=16, causal=False)
    out, lse, flags = run_gpu(torch, M, wl2)
    assert flags & M.MLA_FLAG_BAD_BLOCK
    ref_o, ref_l = oracle(wl)                  # request 0 is untouched
    check(out[0:1], lse[0:1], ref_o[0:1], ref_l[0:1], "request beside a bad block entry")


def test_workspace_without_matching_plan_sets_flag_without_fault(torch, M):
    """A workspace that holds no plan, or a plan made for other parameters: the decode reads no plan entry,
    writes out = 0 and lse = -inf for every row and sets MLA_FLAG_BAD_PLAN; the combine leaves them alone.
    A matching plan afterwards gives the oracle's result again."""
    wl = W.make_workload("badplan", batch=3, num_heads=32, seqlens=[300, 77, 1500], seed=9, spare_pages=2)
    q, kv, _, bt, sl = to_gpu(torch, wl)
    mk = lambda nwg: M.MlaDecode(batch=3, seqlen_q=1, num_heads=32, num_pages=wl.num_pages,
                                 max_blocks_per_seq=wl.block_table.shape[1], num_workgroups=nwg)
    dec, other = mk(5), mk(3)
    assert other.workspace_bytes <= dec.workspace_bytes
    stream = torch.cuda.current_stream().cuda_stream

    def run_unplanned():
        dec.out.fill_(1.0)
        dec.lse.fill_(1.0)
        dec.decode(q, kv, bt, sl)
        dec.combine()
        torch.cuda.synchronize()
        assert dec.flags() & M.MLA_FLAG_BAD_PLAN
        assert (dec.out.float() == 0).all().item()
        assert torch.isneginf(dec.lse).all().item()

    _say("unplanned workspace")
    dec.workspace.zero_()                      # never planned
    run_unplanned()
    _say("plan for another workgroup count")
    M.mla_get_workspace(other.params, sl.data_ptr(), dec.workspace.data_ptr(), dec.workspace_bytes, stream)
    run_unplanned()
    _say("matching plan")
    out, lse = dec(q, kv, bt, sl)
    torch.cuda.synchronize()
    assert dec.flags() == 0
    ref_o, ref_l = oracle(wl)
    check(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref_o, ref_l, "after re-plan")


def test_out_of_range_seqlen_is_clamped_and_flagged(torch, M):
    """A length past the block table's reach is clamped to its pages and flagged; a length of 0 gives an empty
    result.  Request 1 fills its two pages exactly, so every token of the clamped range is finite."""
    wl = W.make_workload("clamp", batch=2, num_heads=16, seqlens=[100, 128], seed=4)
    sl = wl.seqlens.copy()
    sl[1] = 100000                       # beyond max_blocks * 64 = 128
    sl[0] = 0                            # below s_q: an empty request
    wl2 = W.Workload(name="clamp2", q=wl.q, cache=wl.cache, kv_scale=None, block_table=wl.block_table, seqlens=sl,
                     s_q=1, num_heads=16, causal=False)
    out, lse, flags = run_gpu(torch, M, wl2)
    assert flags & M.MLA_FLAG_SEQLEN_CLAMPED
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    ref_o, ref_l = oracle(wl)                  # 100000 clamps to 2 pages = 128 tokens: the original request 1
    assert np.isfinite(ref_o[1]).all()
    check(out[1:2], lse[1:2], ref_o[1:2], ref_l[1:2], "clamped request")


# ------------------------------------------------------------------ full-size configurations, every row
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dsv3_b64_h128_l4096", "ragged_b128_h128_l128_32768", "mtp_b32_h128_sq2_l8192"])
def test_full_config_every_row(torch, M, name):
    """The measured configurations at full size, every output row against the oracle (relative L2 over the
    whole tensor, the worst row reported)."""
    _say(f"full config {name}: generating")
    wl = W.make_config(name)
    _say(f"full config {name}: running on GPU")
    out, lse, flags = run_gpu(torch, M, wl)
    assert flags == 0
    _say(f"full config {name}: oracle on all {wl.batch * wl.s_q * wl.num_heads} rows")
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"{name} (whole tensor)")


@pytest.mark.timeout(600)
def test_single_long_request_split_everywhere(torch, M):
    """One 131,072-token request: every persistent workgroup holds a piece; the combine merges 256 pieces."""
    wl = W.make_workload("long1", batch=1, num_heads=128, seqlens=[131072], seed=8)
    _say("131072-token request")
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, "131072-token request (every row)")
