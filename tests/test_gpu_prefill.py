"""The expand path (prefill / extend) against the fp64 oracle, through the C ABI (MI355X only).

* mla_expand_kv: k^N = W_UK[h] c and v = W_UV[h] c are products of bf16 numbers summed in fp32 over
  K = 512 and rounded once to bf16, so each element satisfies
  |got - ref| <= 2^-8 |ref| + 512 * 2^-23 * sum_c |w c|; the k^R copy and the zero padding are exact.
* mla_prefill_attention on given bf16 K and V^T: the decode kernel's arithmetic and bounds (out max-abs
  2e-2, rel-L2 5e-3, LSE 1e-3); rows that see no key of the range get out 0 and LSE -inf exactly.
* mla_lse_merge: the combine's arithmetic; output within one bf16 rounding, LSE within 1e-5.
* mla_chunked_prefill against the oracle's expand path (expand_attention): the expanded K and V are
  rounded to bf16 before the attention.  The LSE is 1-Lipschitz in the largest score change, and one
  RNE rounding of k (plus its fp32 sum over 512 terms) moves a score by at most
  scale * sum_d |q_d| (2^-9 |k_d| + 512 2^-24 sum_c |w c|), so the LSE bound is 1e-3 plus that with
  both terms doubled, maximised over the keys the row sees;
  the output keeps the decode bounds (a CPU simulation of these roundings gives max-abs 1e-2, rel-L2
  2.8e-3 on these inputs).
"""
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


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")


def _bits(torch, t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def _params(M, pw, chunk):
    return M.make_prefill_params(num_heads=pw.num_heads, num_new=pw.num_new, seqlen=pw.seqlen,
                                 num_pages=pw.num_pages, max_blocks=len(pw.block_table), chunk_tokens=chunk,
                                 softmax_scale=float(pw.softmax_scale))


def _latents(pw):
    c, kr = W.prefill_latents(pw)
    return c.astype(np.float64), kr.astype(np.float64)


# ------------------------------------------------------------------ expansion
@pytest.mark.parametrize("H,L,t0,ntok", [(16, 700, 0, 700), (128, 300, 64, 200), (4, 5000, 1000, 4000),
                                         (8, 130, 129, 1), (3, 1000, 100, 777), (1, 64, 0, 64), (127, 600, 37, 300),
                                         (64, 3300, 250, 3000), (128, 2200, 0, 2200)])
def test_expand_kv_matches_oracle(torch, M, H, L, t0, ntok):
    pw = W.make_prefill_workload("exp", num_heads=H, num_new=1, seqlen=L, seed=H + L + t0)
    _say(f"expand_kv H={H} L={L} t0={t0} ntok={ntok}")
    ld = (ntok + 63) // 64 * 64
    k = torch.full((H, ld, 192), 0x7FC1, dtype=torch.int16, device="cuda")    # NaN: every element must be written
    vt = torch.full((H, 128, ld), 0x7FC1, dtype=torch.int16, device="cuda")
    cache, bt = _dev(torch, pw.cache), _dev(torch, pw.block_table)
    wuk, wuv = _dev(torch, pw.w_uk), _dev(torch, pw.w_uv)
    M.mla_expand_kv(_params(M, pw, 4096), cache.data_ptr(), bt.data_ptr(), t0, ntok, wuk.data_ptr(), wuv.data_ptr(),
                    k.data_ptr(), vt.data_ptr(), torch.cuda.current_stream().cuda_stream)
    kb, vb = _bits(torch, k), _bits(torch, vt)
    assert (kb[:, ntok:] == 0).all() and (vb[:, :, ntok:] == 0).all(), "padding rows must be zero"
    rows = pw.cache[pw.block_table[:(L + 63) // 64]].reshape(-1, 576)[t0:t0 + ntok]
    assert np.array_equal(kb[:, :ntok, 128:], np.broadcast_to(rows[:, 512:], (H, ntok, 64))), "k^R is copied exactly"
    c, kr = _latents(pw)
    c, kr = c[t0:t0 + ntok], kr[t0:t0 + ntok]
    wk, wv = _f64(pw.w_uk), _f64(pw.w_uv)
    ref_k, ref_v = O.expand_kv(c, kr, wk, wv)
    abs_k, abs_v = O.expand_kv(np.abs(c), np.abs(kr), np.abs(wk), np.abs(wv))
    for name, got, ref, ab in (("k^N", _f64(kb[:, :ntok, :128]), ref_k[..., :128], abs_k[..., :128]),
                               ("v", _f64(vb[:, :, :ntok]).transpose(0, 2, 1), ref_v, abs_v)):
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 512 * 2.0 ** -23 * ab
        _say(f"  {name}: max-abs {err.max():.3e} worst err/bound {(err / bound).max():.3f}")
        assert (err <= bound).all(), f"{name}: {(err > bound).sum()} elements over the bound"


# ------------------------------------------------------------------ attention over one range
def _random_kv(rng, H, ntok):
    ld = (ntok + 63) // 64 * 64
    k = np.zeros((H, ld, 192), np.float32)
    v = np.zeros((H, ld, 128), np.float32)
    k[:, :ntok] = rng.standard_normal((H, ntok, 192), dtype=np.float32)
    v[:, :ntok] = rng.standard_normal((H, ntok, 128), dtype=np.float32)
    return W.f32_to_bf16_bits(k), W.f32_to_bf16_bits(v)


def _check_rows(got_o, got_l, ref_o, ref_l, what, lse_bound=None):
    got_o = np.asarray(got_o, np.float64).reshape(ref_o.shape)
    got_l = np.asarray(got_l, np.float64).reshape(ref_l.shape)
    empty = np.isneginf(ref_l)
    assert (np.isneginf(got_l) == empty).all(), f"{what}: rows without visible keys differ"
    assert (got_o[empty] == 0).all(), f"{what}: a row without visible keys must be 0"
    seen = ~empty
    err = np.abs(got_o - ref_o)[seen]
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref_o[seen]), 1e-30)
    lerr = np.abs(got_l[seen] - ref_l[seen])   # only rows that see a key: no -inf - -inf
    lb = LSE_MAX_ABS if lse_bound is None else lse_bound[seen]
    _say(f"{what}: out max-abs {err.max():.3e} rel-L2 {rel:.3e}  lse max-abs {lerr.max():.3e} "
         f"(worst lse err/bound {(lerr / lb).max():.3f}; {empty.sum()} empty rows)")
    assert err.max() <= OUT_MAX_ABS and rel <= OUT_REL_L2
    assert (lerr <= lb).all()


@pytest.mark.parametrize("H,n,L,t0,ntok", [(16, 200, 1000, 0, 1000), (16, 130, 1000, 640, 360),
                                           (8, 100, 1000, 950, 50), (128, 64, 64, 0, 64), (4, 300, 5000, 1024, 1500),
                                           (2, 1, 77, 0, 77), (8, 600, 2000, 1400, 600), (16, 520, 1800, 0, 1800)])
def test_prefill_attention_matches_oracle(torch, M, H, n, L, t0, ntok):
    rng = np.random.default_rng(H * 1000 + n + t0)
    q = W.f32_to_bf16_bits(rng.standard_normal((n, H, 192), dtype=np.float32))
    kbits, vbits = _random_kv(rng, H, ntok)
    _say(f"prefill attention H={H} n={n} L={L} t0={t0} ntok={ntok}")
    p = M.make_prefill_params(num_heads=H, num_new=n, seqlen=L, num_pages=(L + 63) // 64,
                              max_blocks=(L + 63) // 64, chunk_tokens=4096)
    qd, kd = _dev(torch, q), _dev(torch, kbits)
    vtd = _dev(torch, np.ascontiguousarray(vbits.transpose(0, 2, 1)))
    out = torch.empty((n, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((n, H), dtype=torch.float32, device="cuda")
    M.mla_prefill_attention(p, qd.data_ptr(), kd.data_ptr(), vtd.data_ptr(), t0, ntok, out.data_ptr(),
                            lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref_o, ref_l = O.mha_attend(_f64(q), _f64(kbits[:, :ntok]), _f64(vbits[:, :ntok]), float(p.softmax_scale),
                                np.arange(L - n, L), np.arange(t0, t0 + ntok))
    _check_rows(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "attention")


# ------------------------------------------------------------------ merge
def test_lse_merge_matches_oracle(torch, M):
    rng = np.random.default_rng(5)
    J, R = 5, 1000
    parts = rng.standard_normal((J, R, 128)).astype(np.float32)
    lparts = (rng.standard_normal((J, R)) * 3).astype(np.float32)
    lparts[rng.random((J, R)) < 0.3] = -np.inf
    lparts[:, 17] = -np.inf                      # a row no part covers
    _say("lse merge J=5 R=1000")
    out = torch.empty((R, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((R,), dtype=torch.float32, device="cuda")
    pd, ld = _dev(torch, parts), _dev(torch, lparts)
    M.mla_lse_merge(R, J, pd.data_ptr(), ld.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    torch.cuda.current_stream().cuda_stream)
    got = _f64(_bits(torch, out))
    got_l = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = O.lse_merge(parts.astype(np.float64), lparts.astype(np.float64))
    assert (got[17] == 0).all() and np.isneginf(got_l[17])
    ok = np.isfinite(ref_l)
    assert np.isneginf(got_l[~ok]).all()
    assert (np.abs(got - ref_o)[ok] <= 2.0 ** -8 * np.abs(ref_o[ok]) + 1e-5).all()
    assert np.abs(got_l[ok] - ref_l[ok]).max() <= 1e-5


# ------------------------------------------------------------------ the whole expand path
def _run_chunked(torch, M, pw, chunk):
    pre = M.MlaPrefill(num_heads=pw.num_heads, num_new=pw.num_new, seqlen=pw.seqlen, num_pages=pw.num_pages,
                       max_blocks=len(pw.block_table), chunk_tokens=chunk, softmax_scale=float(pw.softmax_scale))
    out, lse = pre(_dev(torch, pw.q), _dev(torch, pw.cache), _dev(torch, pw.block_table), _dev(torch, pw.w_uk),
                   _dev(torch, pw.w_uv))
    return _bits(torch, out), lse.cpu().numpy()


def _oracle_expand(pw, rows=None, heads=None):
    """expand_attention for the request; optionally only some query rows and heads (independent per head)."""
    heads = np.arange(pw.num_heads) if heads is None else np.asarray(heads)
    rows = np.arange(pw.num_new) if rows is None else np.asarray(rows)
    L, n = pw.seqlen, pw.num_new
    q = _f64(pw.q)[rows][:, heads]
    wk, wv = _f64(pw.w_uk)[heads], _f64(pw.w_uv)[heads]
    c, kr = _latents(pw)
    qpos, kpos = L - n + rows, np.arange(L)
    out, lse = O.expand_attention(q[..., :128], q[..., 128:], wk, wv, c, kr, float(pw.softmax_scale), qpos, kpos)
    # LSE bound from the bf16 rounding of the expanded keys: |bf16(k) - k| <= 2^-9 |k| plus the fp32
    # accumulation of k (512 terms), both doubled.
    k, _ = O.expand_kv(c, kr, wk, wv)
    kabs, _ = O.expand_kv(np.abs(c), np.abs(kr), np.abs(wk), np.abs(wv))
    absdot = np.einsum("qhd,htd->qht", np.abs(q), 2.0 ** -8 * np.abs(k) + 512 * 2.0 ** -23 * kabs)
    absdot = np.where((kpos[None, :] <= qpos[:, None])[:, None, :], absdot, 0.0)
    bound = LSE_MAX_ABS + float(pw.softmax_scale) * absdot.max(axis=-1)
    return out, lse, bound


@pytest.mark.parametrize("H,n,L,chunk", [(16, 200, 1500, 256), (16, 300, 300, 128), (16, 300, 300, 4096),
                                         (8, 64, 4000, 1024), (16, 1, 500, 128), (128, 96, 700, 256),
                                         (5, 100, 900, 320)])
def test_chunked_prefill_matches_expand_path(torch, M, H, n, L, chunk):
    pw = W.make_prefill_workload("pf", num_heads=H, num_new=n, seqlen=L, seed=3 * H + n + L)
    _say(f"chunked prefill H={H} n={n} L={L} chunk={chunk}")
    out, lse = _run_chunked(torch, M, pw, chunk)
    ref_o, ref_l, lb = _oracle_expand(pw)
    _check_rows(_f64(out), lse, ref_o, ref_l, f"chunked H={H} n={n} L={L} chunk={chunk}", lse_bound=lb)


def test_chunk_size_does_not_change_the_result_beyond_rounding(torch, M):
    pw = W.make_prefill_workload("pf", num_heads=8, num_new=150, seqlen=2000, seed=77)
    _say("chunk sizes 64 / 640 / 4096")
    runs = [_run_chunked(torch, M, pw, c) for c in (64, 640, 4096)]
    ref_o, ref_l, lb = _oracle_expand(pw)
    for (o, l), c in zip(runs, (64, 640, 4096)):
        _check_rows(_f64(o), l, ref_o, ref_l, f"chunk={c}", lse_bound=lb)


def test_prefill_block_table_permutation_is_bit_exact(torch, M):
    pw = W.make_prefill_workload("perm", num_heads=8, num_new=100, seqlen=1000, seed=12, spare_pages=5)
    o1, l1 = _run_chunked(torch, M, pw, 256)
    P = pw.num_pages
    perm = np.random.default_rng(99).permutation(P).astype(np.int32)
    cache2 = np.empty_like(pw.cache)
    cache2[perm] = pw.cache
    bt2 = np.where(pw.block_table >= 0, perm[np.maximum(pw.block_table, 0)], -1).astype(np.int32)
    pw2 = W.PrefillWorkload(name="perm2", q=pw.q, cache=cache2, block_table=bt2, w_uk=pw.w_uk, w_uv=pw.w_uv,
                            seqlen=pw.seqlen, num_new=pw.num_new, num_heads=pw.num_heads)
    o2, l2 = _run_chunked(torch, M, pw2, 256)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("chunk", [8192, 33280])
def test_extend_after_32k_prefix_sampled(torch, M, chunk):
    """The handbook's "+512 new tokens after a 32K prefix" at 128 heads, in chunks of 8,192 and as one chunk of
    the whole context: the GPU computes everything; the oracle computes 3 query rows of 2 heads."""
    pw = W.make_prefill_workload("extend", num_heads=128, num_new=512, seqlen=32768 + 512, seed=8)
    _say(f"extend 32K + 512, H=128, chunk {chunk} (sampled)")
    out, lse = _run_chunked(torch, M, pw, chunk)
    rows, heads = np.array([0, 256, 511]), np.array([5, 127])
    ref_o, ref_l, lb = _oracle_expand(pw, rows=rows, heads=heads)
    got_o = _f64(out)[rows][:, heads]
    got_l = lse[rows][:, heads]
    _check_rows(got_o, got_l, ref_o, ref_l, "extend sampled", lse_bound=lb)


@pytest.mark.parametrize("H,n,L", [(16, 300, 300), (8, 150, 2000), (128, 40, 700)])
def test_single_chunk_equals_expand_attend_merge(torch, M, H, n, L):
    """A call whose one chunk covers the context skips the merge: its bf16 rows and LSEs must be bit-identical to
    expansion, attention into an fp32 part and a merge of that single part, run as separate calls."""
    pw = W.make_prefill_workload("one", num_heads=H, num_new=n, seqlen=L, seed=H + n + L)
    _say(f"single chunk vs expand/attend/merge H={H} n={n} L={L}")
    o1, l1 = _run_chunked(torch, M, pw, -(-L // 64) * 64)
    p = _params(M, pw, -(-L // 64) * 64)
    ld = -(-L // 64) * 64
    s = torch.cuda.current_stream().cuda_stream
    cache, bt = _dev(torch, pw.cache), _dev(torch, pw.block_table)
    wuk, wuv, q = _dev(torch, pw.w_uk), _dev(torch, pw.w_uv), _dev(torch, pw.q)
    k = torch.empty((H, ld, 192), dtype=torch.int16, device="cuda")
    vt = torch.empty((H, 128, ld), dtype=torch.int16, device="cuda")
    part = torch.empty((n, H, 128), dtype=torch.float32, device="cuda")
    lpart = torch.empty((n, H), dtype=torch.float32, device="cuda")
    out = torch.empty((n, H, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((n, H), dtype=torch.float32, device="cuda")
    M.mla_expand_kv(p, cache.data_ptr(), bt.data_ptr(), 0, L, wuk.data_ptr(), wuv.data_ptr(), k.data_ptr(),
                    vt.data_ptr(), s)
    M.mla_prefill_attention(p, q.data_ptr(), k.data_ptr(), vt.data_ptr(), 0, L, part.data_ptr(), lpart.data_ptr(), s)
    M.mla_lse_merge(n * H, 1, part.data_ptr(), lpart.data_ptr(), out.data_ptr(), lse.data_ptr(), s)
    o2, l2 = _bits(torch, out), lse.cpu().numpy()
    assert np.array_equal(o1.reshape(-1), o2.reshape(-1))
    assert np.array_equal(l1.reshape(-1).view(np.uint32), l2.reshape(-1).view(np.uint32))
