"""The two projections of the absorb path against the fp64 oracle, through the C
ABI (MI355X only), and the whole absorb path (absorb -> decode -> combine ->
output projection) against the oracle's expand path.

Projection bound, element by element: the kernels multiply bf16 numbers exactly
in fp32, accumulate K of them in fp32 and round once to bf16, so
    |got - ref| <= 2^-8 |ref| + K 2^-23 sum_k |a_k b_k|
(one round-to-nearest bf16 rounding, unit 2^-8, plus a K-term fp32 sum with
unit 2^-24, doubled for slack).  The q^R copy is bit-exact.

End-to-end bound: the absorb path rounds q~ and the latent output to bf16 on
top of what the decode does.  Those two roundings alone, applied to fp64
arithmetic on these inputs, move the output by rel-L2 ~3.3e-3 (max-abs ~8e-3)
and the LSE by ~3.6e-3 against the expand path; with the decode's own budget
(rel-L2 5e-3) that gives rel-L2 <= 1e-2, max-abs <= 3e-2, LSE max-abs <= 1e-2.
"""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

E2E_REL_L2 = 1e-2
E2E_MAX_ABS = 3e-2
E2E_LSE_MAX_ABS = 1e-2


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


def _dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def _host_bits(torch, t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def _check_bound(got_bits, ref, absref, K, what):
    got = _f64(got_bits)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -23 * absref
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _say(f"{what}: max-abs {err.max():.3e}  worst err/bound {(err / bound).max():.3f}  rel-L2 {rel:.3e}")
    assert (err <= bound).all(), f"{what}: {(err > bound).sum()} elements over the bound"
    assert rel <= 2.0 ** -8, f"{what}: rel-L2 {rel}"


def _run_absorb(torch, M, pi):
    q_tilde = M.absorb_q(_dev(torch, pi.q_nope), _dev(torch, pi.q_rope), _dev(torch, pi.w_uk))
    return _host_bits(torch, q_tilde)


def _run_project(torch, M, o_bits, w_uv_bits):
    return _host_bits(torch, M.project_out(_dev(torch, o_bits), _dev(torch, w_uv_bits)))


@pytest.mark.parametrize("T,H", [(1, 1), (16, 16), (17, 128), (64, 128), (300, 128), (33, 5)])
def test_absorb_q_matches_oracle(torch, M, T, H):
    pi = W.make_proj_inputs(tokens=T, num_heads=H, seed=T * 131 + H)
    _say(f"absorb_q T={T} H={H}")
    got = _run_absorb(torch, M, pi)
    assert got.shape == (T, H, 576)
    assert np.array_equal(got[..., 512:], pi.q_rope), "q^R must be copied bit for bit"
    qn, wuk = _f64(pi.q_nope), _f64(pi.w_uk)
    ref = O.absorb_q(qn, _f64(pi.q_rope), wuk)[..., :512]
    absref = O.absorb_q(np.abs(qn), np.zeros((T, H, 64)), np.abs(wuk))[..., :512]
    _check_bound(got[..., :512], ref, absref, 128, f"absorb T={T} H={H}")


@pytest.mark.parametrize("T,H", [(1, 1), (16, 16), (17, 128), (64, 128), (300, 128), (33, 5)])
def test_project_out_matches_oracle(torch, M, T, H):
    pi = W.make_proj_inputs(tokens=1, num_heads=H, seed=T * 17 + H)
    rng = np.random.default_rng(T + 1000 * H)
    o_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H, 512), dtype=np.float32) * np.float32(0.3))
    _say(f"project_out T={T} H={H}")
    got = _run_project(torch, M, o_bits, pi.w_uv)
    assert got.shape == (T, H, 128)
    o, wuv = _f64(o_bits), _f64(pi.w_uv)
    _check_bound(got, O.project_out(o, wuv), O.project_out(np.abs(o), np.abs(wuv)), 512, f"project T={T} H={H}")


def test_projections_at_many_rows_sampled(torch, M):
    """T = 2,048 rows (32 row tiles per workgroup) at 128 heads; the oracle computes 40 sampled rows."""
    T, H = 2048, 128
    pi = W.make_proj_inputs(tokens=T, num_heads=H, seed=77)
    rng = np.random.default_rng(78)
    o_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H, 512), dtype=np.float32) * np.float32(0.3))
    _say("projections T=2048 H=128 sampled")
    qt = _run_absorb(torch, M, pi)
    out = _run_project(torch, M, o_bits, pi.w_uv)
    rows = np.unique(np.concatenate([[0, 15, 16, T - 17, T - 1], rng.choice(T, 35, replace=False)]))
    assert np.array_equal(qt[..., 512:], pi.q_rope)
    qn, wuk, wuv, o = _f64(pi.q_nope[rows]), _f64(pi.w_uk), _f64(pi.w_uv), _f64(o_bits[rows])
    _check_bound(qt[rows, :, :512], O.absorb_q(qn, _f64(pi.q_rope[rows]), wuk)[..., :512],
                 O.absorb_q(np.abs(qn), np.zeros((len(rows), H, 64)), np.abs(wuk))[..., :512], 128, "absorb sampled")
    _check_bound(out[rows], O.project_out(o, wuv), O.project_out(np.abs(o), np.abs(wuv)), 512, "project sampled")


def test_projection_writes_stay_in_place(torch, M):
    """Guard regions around q~ and out are untouched; inputs are not written."""
    T, H = 19, 7
    pi = W.make_proj_inputs(tokens=T, num_heads=H, seed=5)
    qn, qr, wuk, wuv = (_dev(torch, x) for x in (pi.q_nope, pi.q_rope, pi.w_uk, pi.w_uv))
    guard = 4096
    qt_buf = torch.full((guard + T * H * 576 + guard,), 0x7FC1, dtype=torch.int16, device="cuda")
    qt = qt_buf[guard:guard + T * H * 576].view(T, H, 576)
    M.absorb_q(qn, qr, wuk, out=qt)
    o = qt[..., :512].contiguous()
    out_buf = torch.full((guard + T * H * 128 + guard,), 0x7FC1, dtype=torch.int16, device="cuda")
    M.project_out(o, wuv, out=out_buf[guard:guard + T * H * 128].view(T, H, 128))
    torch.cuda.synchronize()
    for buf, n in ((qt_buf, T * H * 576), (out_buf, T * H * 128)):
        h = buf.cpu().numpy()
        assert (h[:guard] == 0x7FC1).all() and (h[guard + n:] == 0x7FC1).all()
    for dev, bits in ((qn, pi.q_nope), (qr, pi.q_rope), (wuk, pi.w_uk), (wuv, pi.w_uv)):
        assert np.array_equal(_host_bits(torch, dev), bits)


# ------------------------------------------------------------------ the whole absorb path vs the expand path
@pytest.mark.parametrize("seqlens,s_q,nwg", [([300, 77, 1500], 1, 0), ([200, 900], 2, 0), ([4096, 4096], 1, 0),
                                             ([300, 77, 1500], 1, 7)])
def test_absorb_path_equals_expand_path(torch, M, seqlens, s_q, nwg):
    """absorb_q -> mla_decode_fwd (+ combine) -> project_out on the GPU against the
    oracle's expand path (per-head keys and values rebuilt from the latent)."""
    H = 128
    B, T = len(seqlens), len(seqlens) * s_q
    seed = sum(seqlens) + s_q
    wl = W.make_workload("e2e", batch=B, num_heads=H, seqlens=seqlens, s_q=s_q, causal=s_q > 1, seed=seed,
                         spare_pages=3)
    pi = W.make_proj_inputs(tokens=T, num_heads=H, seed=seed + 1)
    _say(f"absorb path seqlens={seqlens} s_q={s_q} nwg={nwg}")
    kv = torch.from_numpy(wl.cache.view(np.int16)).to("cuda")
    bt = torch.from_numpy(wl.block_table).to("cuda")
    sl = torch.from_numpy(wl.seqlens).to("cuda")
    q_tilde = M.absorb_q(_dev(torch, pi.q_nope), _dev(torch, pi.q_rope), _dev(torch, pi.w_uk))
    dec = M.MlaDecode(batch=B, seqlen_q=s_q, num_heads=H, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], causal=wl.causal, kv_dtype=M.MLA_KV_BF16,
                      softmax_scale=float(wl.softmax_scale), num_workgroups=nwg)
    o, lse = dec(q_tilde.view(B, s_q, H, 576), kv, bt, sl, None)
    out = M.project_out(o.view(T, H, 512), _dev(torch, pi.w_uv))
    got = _f64(_host_bits(torch, out)).reshape(B, s_q, H, 128)
    lse = lse.cpu().numpy().astype(np.float64).reshape(B, s_q, H)

    qn, qr, wuk, wuv = (_f64(x) for x in (pi.q_nope, pi.q_rope, pi.w_uk, pi.w_uv))
    errs, refs, lerrs = [], [], []
    for b, L in enumerate(seqlens):
        pages = wl.block_table[b, :(L + 63) // 64]
        c = _f64(wl.cache[pages].reshape(-1, 576)[:L])
        rows = slice(b * s_q, (b + 1) * s_q)
        ref, ref_lse = O.expand_attention(qn[rows], qr[rows], wuk, wuv, c[:, :512], c[:, 512:],
                                          float(wl.softmax_scale), np.arange(L - s_q, L), np.arange(L))
        errs.append(got[b] - ref)
        refs.append(ref)
        lerrs.append(lse[b] - ref_lse)
    err, ref, lerr = np.concatenate(errs), np.concatenate(refs), np.concatenate(lerrs)
    rel = np.linalg.norm(err) / np.linalg.norm(ref)
    _say(f"  out max-abs {np.abs(err).max():.3e} rel-L2 {rel:.3e}  lse max-abs {np.abs(lerr).max():.3e}")
    assert np.isfinite(got).all()
    assert rel <= E2E_REL_L2
    assert np.abs(err).max() <= E2E_MAX_ABS
    assert np.abs(lerr).max() <= E2E_LSE_MAX_ABS
