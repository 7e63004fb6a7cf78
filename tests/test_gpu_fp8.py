"""FP8 (E4M3FN codes + one fp32 scale per token) HIP path vs the fp64 oracle (MI355X only).

The oracle decodes each code exactly and multiplies by its scale in fp64.  The
kernel widens codes to bf16 exactly and applies the scale in fp32 to the score
and to the softmax weight before the weight is rounded to bf16, so the error
budget is the bf16 path's: the same tolerances apply.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import OUT_MAX_ABS, _say, check, oracle, run_gpu

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


def _fp8(name, **kw):
    return W.make_workload(name, kv_dtype="fp8_e4m3fn", **kw)


def test_fp8_small(torch, M):
    wl = _fp8("fp8small", batch=2, num_heads=16, seqlens=[256, 97], seed=41, spare_pages=2)
    _say("fp8 small")
    out, lse, flags = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, "fp8 small")
    assert flags == 0


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 63, 64, 65, 129, 1000])
def test_fp8_lengths_with_poison(torch, M, L):
    """Scales and codes past each request's end are NaN; none of it may reach the output."""
    wl = _fp8(f"fp8L{L}", batch=2, num_heads=128, seqlens=[L, L + 3], seed=200 + L, spare_pages=2, poison=True)
    _say(f"fp8 L={L}")
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"fp8 L={L}")


@pytest.mark.parametrize("nwg", [1, 3, 16, 256])
def test_fp8_split_invariance(torch, M, nwg):
    wl = _fp8("fp8splits", batch=4, num_heads=128, seqlens=[64, 700, 2049, 130], seed=43, spare_pages=3)
    _say(f"fp8 split invariance nwg={nwg}")
    out, lse, _ = run_gpu(torch, M, wl, num_workgroups=nwg)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"fp8 nwg={nwg}")


@pytest.mark.parametrize("H,s_q", [(16, 1), (64, 2), (128, 2), (20, 3), (128, 8)])
def test_fp8_heads_and_new_tokens(torch, M, H, s_q):
    wl = _fp8(f"fp8h{H}s{s_q}", batch=3, num_heads=H, seqlens=[300, 77, 1500], s_q=s_q, causal=s_q > 1,
              seed=50 + H + s_q, spare_pages=2)
    _say(f"fp8 H={H} s_q={s_q}")
    out, lse, _ = run_gpu(torch, M, wl)
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"fp8 H={H} s_q={s_q}")


def test_fp8_block_table_permutation_is_bit_exact(torch, M):
    wl = _fp8("fp8perm", batch=3, num_heads=128, seqlens=[1000, 64, 333], seed=44, spare_pages=5)
    out1, lse1, _ = run_gpu(torch, M, wl)
    rng = np.random.default_rng(7)
    perm = rng.permutation(wl.num_pages).astype(np.int32)
    cache2 = np.empty_like(wl.cache)
    cache2[perm] = wl.cache
    scale2 = np.empty_like(wl.kv_scale)
    scale2[perm] = wl.kv_scale
    bt2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    wl2 = W.Workload(name="fp8perm2", q=wl.q, cache=cache2, kv_scale=scale2, block_table=bt2, seqlens=wl.seqlens,
                     s_q=wl.s_q, num_heads=wl.num_heads, causal=wl.causal)
    out2, lse2, _ = run_gpu(torch, M, wl2)
    assert np.array_equal(out1, out2)
    assert np.array_equal(lse1.view(np.uint32), lse2.view(np.uint32))


def test_fp8_scale_is_applied_per_token(torch, M):
    """Doubling every scale of one request doubles every cached value: compare both against the oracle, which
    takes the scales as given.  The doubled cache doubles the outputs and so the bf16 rounding error of each
    output element (relative 2^-9), so its max-abs bound is the bf16 bound times 2; the relative L2 and LSE
    bounds are unchanged (the FP8 bar itself is relative L2 <= 3e-2)."""
    wl = _fp8("fp8scale", batch=1, num_heads=16, seqlens=[200], seed=45, spare_pages=1)
    ks = wl.kv_scale.copy()
    ks[np.isfinite(ks)] *= 2.0
    wl2 = W.Workload(name="fp8scale2", q=wl.q, cache=wl.cache, kv_scale=ks, block_table=wl.block_table,
                     seqlens=wl.seqlens, s_q=1, num_heads=16, causal=False)
    for w, factor in ((wl, 1.0), (wl2, 2.0)):
        out, lse, _ = run_gpu(torch, M, w)
        ref_o, ref_l = oracle(w)
        check(out, lse, ref_o, ref_l, w.name, max_abs=OUT_MAX_ABS * factor)


@pytest.mark.timeout(900)
def test_fp8_full_config_every_row(torch, M):
    """The FP8 configuration at full size (128 requests x 16,384 tokens), every output row against the oracle."""
    name = "fp8_b128_h128_l16384"
    _say(f"full config {name}: generating")
    wl = W.make_config(name)
    _say(f"full config {name}: running on GPU")
    out, lse, flags = run_gpu(torch, M, wl)
    assert flags == 0
    _say(f"full config {name}: oracle on all {wl.batch * wl.num_heads} rows")
    ref_o, ref_l = oracle(wl)
    check(out, lse, ref_o, ref_l, f"{name} (whole tensor)")
