"""The FP8-MFMA route (MLA_FP8_PATH_MFMA) against the exact fp64 oracle (MI355X only).

The route rounds q~ to a per-row scale times a sum of two E4M3 numbers (about 2^-8 of q~) and each softmax
weight times its token's scale to E4M3 (3 mantissa bits) for the value product, so it is compared at the
metric's FP8 bound: relative L2 <= 3e-2 over the output (whole tensor; on random inputs it measures about
1.5e-2, where the exact FP8 route measures 2e-3).  The LSE carries only the score's error from q~
(~2^-8 relative) and fp32 sums: bound 1e-2.  Block-table indexing stays bit-exact: a permuted physical page
layout gives identical bits.  The 128-token chunk of this route puts the length edges at 127/128/129.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _say, oracle, run_gpu

pytestmark = pytest.mark.gpu

REL_L2 = 3e-2
LSE_MAX_ABS = 1e-2
MFMA = 1   # MLA_FP8_PATH_MFMA


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


def _fp8(name, **kw):
    return W.make_workload(name, kv_dtype="fp8_e4m3fn", **kw)


def check_route(out_bits, lse, ref_out, ref_lse, what):
    got = W.bf16_bits_to_f32(out_bits).astype(np.float64).reshape(ref_out.shape)
    lse = np.asarray(lse, np.float64).reshape(ref_lse.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = (got - ref_out).reshape(-1, got.shape[-1])
    r = ref_out.reshape(-1, got.shape[-1])
    rel = np.linalg.norm(d) / max(np.linalg.norm(r), 1e-30)
    row_rel = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    lerr = np.abs(lse - ref_lse)
    _say(f"{what}: out rel-L2 {rel:.3e} (worst row {row_rel.max():.3e}), max-abs {np.abs(d).max():.3e}, "
         f"lse max-abs {lerr.max():.3e}  [{d.shape[0]} rows]")
    assert rel <= REL_L2, f"{what}: out rel-L2 {rel}"
    assert lerr.max() <= LSE_MAX_ABS, f"{what}: lse max-abs {lerr.max()}"


def test_mfma_route_small(torch, M):
    wl = _fp8("f8m-small", batch=2, num_heads=16, seqlens=[256, 97], seed=61, spare_pages=2)
    out, lse, flags = run_gpu(torch, M, wl, fp8_path=MFMA)
    ref_o, ref_l = oracle(wl)
    check_route(out, lse, ref_o, ref_l, "fp8-mfma small")
    assert flags == 0


@pytest.mark.parametrize("L", [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000])
def test_mfma_route_lengths_with_poison(torch, M, L):
    """Codes and scales past each request's end are NaN; none of it may reach the output."""
    wl = _fp8(f"f8mL{L}", batch=2, num_heads=128, seqlens=[L, L + 3], seed=300 + L, spare_pages=2, poison=True)
    out, lse, _ = run_gpu(torch, M, wl, fp8_path=MFMA)
    ref_o, ref_l = oracle(wl)
    check_route(out, lse, ref_o, ref_l, f"fp8-mfma L={L}")


@pytest.mark.parametrize("nwg", [1, 3, 16, 256])
def test_mfma_route_split_invariance(torch, M, nwg):
    wl = _fp8("f8m-splits", batch=4, num_heads=128, seqlens=[64, 700, 2049, 130], seed=63, spare_pages=3)
    out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg, fp8_path=MFMA)
    ref_o, ref_l = oracle(wl)
    check_route(out, lse, ref_o, ref_l, f"fp8-mfma nwg={nwg}")


@pytest.mark.parametrize("H,s_q", [(16, 1), (64, 2), (128, 2), (20, 3), (128, 8)])
def test_mfma_route_heads_and_new_tokens(torch, M, H, s_q):
    wl = _fp8(f"f8m-h{H}s{s_q}", batch=3, num_heads=H, seqlens=[300, 77, 1500], s_q=s_q, causal=s_q > 1,
              seed=70 + H + s_q, spare_pages=2)
    out, lse, _ = run_gpu(torch, M, wl, fp8_path=MFMA)
    ref_o, ref_l = oracle(wl)
    check_route(out, lse, ref_o, ref_l, f"fp8-mfma H={H} s_q={s_q}")


JUMP_SEQLENS = [1600, 900, 1100, 2000, 1800]
JUMP_SPANS = [[(1200, 3, 1)], [(896, 3, 1)], [(0, 3, 1)], [(600, 1, 1), (1300, 1, 1), (1999, 1, 1)],
              [(1000, 3, 1), (1700, 1, 2)]]


@pytest.mark.parametrize("nwg", [0, 1, 7])
def test_mfma_route_score_jump_rescales_mid_chunk(torch, M, nwg):
    """Scores that rise partway through a 128-token chunk: the weights gathered so far are folded into O
    before the rescale (earlier keys still carry ~40% of the softmax mass)."""
    wl = W.make_score_jump_workload("f8m-jump", seqlens=JUMP_SEQLENS, jumps=JUMP_SPANS, seed=81,
                                    kv_dtype="fp8_e4m3fn")
    out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg, fp8_path=MFMA)
    ref_o, ref_l = oracle(wl)
    check_route(out, lse, ref_o, ref_l, f"fp8-mfma jump nwg={nwg}")


def test_mfma_route_block_table_permutation_is_bit_exact(torch, M):
    wl = _fp8("f8m-perm", batch=3, num_heads=128, seqlens=[1000, 64, 333], seed=64, spare_pages=5)
    out1, lse1, _ = run_gpu(torch, M, wl, fp8_path=MFMA)
    rng = np.random.default_rng(9)
    perm = rng.permutation(wl.num_pages).astype(np.int32)
    cache2 = np.empty_like(wl.cache)
    cache2[perm] = wl.cache
    scale2 = np.empty_like(wl.kv_scale)
    scale2[perm] = wl.kv_scale
    bt2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    wl2 = W.Workload(name="f8m-perm2", q=wl.q, cache=cache2, kv_scale=scale2, block_table=bt2, seqlens=wl.seqlens,
                     s_q=wl.s_q, num_heads=wl.num_heads, causal=wl.causal)
    out2, lse2, _ = run_gpu(torch, M, wl2, fp8_path=MFMA)
    assert np.array_equal(out1, out2)
    assert np.array_equal(lse1.view(np.uint32), lse2.view(np.uint32))


def test_mfma_route_odd_page_segment_start(torch, M):
    """Split boundaries on odd pages: a segment's 128-token chunks start at any page."""
    wl = _fp8("f8m-odd", batch=2, num_heads=128, seqlens=[64 * 13 + 5, 64 * 7], seed=65, spare_pages=2)
    for nwg in (2, 3, 5, 9):
        out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg, fp8_path=MFMA)
        ref_o, ref_l = oracle(wl)
        check_route(out, lse, ref_o, ref_l, f"fp8-mfma odd segments nwg={nwg}")


@pytest.mark.timeout(900)
def test_mfma_route_full_config_every_row(torch, M):
    """The FP8 configuration (128 requests x 16,384 tokens) on the E4M3 route, every output row."""
    name = "fp8_b128_h128_l16384"
    wl = W.make_config(name)
    _say(f"full config {name} on the FP8-MFMA route")
    out, lse, flags = run_gpu(torch, M, wl, fp8_path=MFMA)
    assert flags == 0
    ref_o, ref_l = oracle(wl)
    check_route(out, lse, ref_o, ref_l, f"{name} fp8-mfma (whole tensor)")
