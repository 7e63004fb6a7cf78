"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics fix:
the expand path (an independent NumPy implementation of the other algorithm the
handbook shows to be equivalent), closed forms, invariants and special cases.
Together they are chosen so a plausible slip in the oracle fails at least one:

  dropped RoPE term / wrong width      -> all-ones closed form, expand == absorb
  wrong softmax scale                  -> all-ones closed form, expand == absorb
  value taken from the wrong slice     -> seqlen-1 exact copy, expand == absorb
  block/slot swapped in the page walk  -> expand == absorb through permuted pages
  wrong causal offset                  -> causal expand == absorb, visibility test
  LSE off by the max / wrong base      -> seqlen-2 closed form, q~ = 0 case
  unnormalised softmax                 -> constant-column test, equal-token case
  broken split merge                   -> split-and-merge == unsplit
  FP8 decode slip                      -> all 256 codes vs torch's float8_e4m3fn
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O

SCALE = float(W.SOFTMAX_SCALE)


def _paged(latent, rope, rng, page=64, spare=3):
    """Scatter logical tokens [T, dc] / [T, dr] into a permuted paged bf16 cache."""
    T = latent.shape[0]
    npg = (T + page - 1) // page
    P = npg + spare
    perm = rng.permutation(P).astype(np.int32)
    cache = np.full((P, page, latent.shape[1] + rope.shape[1]), W.BF16_NAN, dtype=np.uint16)
    bt = perm[:npg][None, :].copy()
    for t in range(T):
        cache[bt[0, t // page], t % page, :latent.shape[1]] = W.f32_to_bf16_bits(latent[t])
        cache[bt[0, t // page], t % page, latent.shape[1]:] = W.f32_to_bf16_bits(rope[t])
    return cache, bt


def _bf16_exact(rng, shape, std=1.0):
    """float64 values that are exactly representable in bf16."""
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)).astype(np.float64)


# ---------------------------------------------------------------- formats
def test_bf16_widening_matches_numpy():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 2000, dtype=np.uint16)
    ref = W.bf16_bits_to_f32(bits).astype(np.float64)
    got = np.array([O.bf16_to_f64(b) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3fn_decode_all_codes_matches_torch(golden):
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3fn_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # the page's facts: largest finite magnitude 448, no infinities
    assert np.nanmax(np.abs(got)) == golden["fp8_formats"]["e4m3_max"]
    assert not np.isinf(got).any()
    assert np.isnan(got).sum() == 2      # S.1111.111 for both signs


# ---------------------------------------------------------------- expand == absorb
def _expand_vs_absorb(rng, H, T, s_q, causal, dc, dr, dn, dv, page=64):
    """Draw tiny W_UK/W_UV and a paged cache; run both paths; return max errors."""
    latent = _bf16_exact(rng, (T, dc))
    rope = _bf16_exact(rng, (T, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)     # k^N = W_UK[h] c
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    q_nope = rng.standard_normal((s_q, H, dn))
    q_rope = rng.standard_normal((s_q, H, dr))
    scale = 1.0 / math.sqrt(dn + dr)

    key_pos = np.arange(T)
    query_pos = np.arange(T - s_q, T) if causal else np.full(s_q, T - 1)
    out_exp, lse_exp = O.expand_attention(q_nope, q_rope, w_uk, w_uv, latent, rope, scale, query_pos, key_pos)

    # absorb: q~ = [W_UK[h]^T q^N ; q^R], latent-space attention, then W_UV (the
    # oracle's absorb_q and project_out, so these pins cover them too)
    q_tilde = O.absorb_q(q_nope, q_rope, w_uk)[None]                   # [1, s_q, H, dc+dr]
    cache, bt = _paged(latent, rope, rng, page=page)
    o_lat, lse_abs = O.attend(q_tilde, cache, bt, np.array([T], np.int32), softmax_scale=np.float32(scale),
                              causal=causal, d_rope=dr)
    out_abs = O.project_out(o_lat[0], w_uv)
    # the oracle takes the scale as fp32; the expand path used the exact double.
    # Compare against an expand run at the same fp32-rounded scale:
    out_exp32, lse_exp32 = O.expand_attention(q_nope, q_rope, w_uk, w_uv, latent, rope,
                                              float(np.float32(scale)), query_pos, key_pos)
    return (np.abs(out_abs - out_exp32).max(), np.abs(lse_abs[0] - lse_exp32).max(),
            np.abs(out_exp32 - out_exp).max())


def test_expand_equals_absorb_deepseek_shapes():
    """Tiny-config shapes (16 heads, 128x512 W_UK/W_UV, seqlen 256, permuted pages): <= 1e-10."""
    rng = np.random.default_rng(11)
    e_out, e_lse, _ = _expand_vs_absorb(rng, H=16, T=256, s_q=1, causal=False, dc=512, dr=64, dn=128, dv=128)
    assert e_out <= 1e-10 and e_lse <= 1e-10, (e_out, e_lse)


def test_expand_equals_absorb_ragged_tail_causal():
    """Two new tokens with the causal mask, a length that ends mid-page."""
    rng = np.random.default_rng(12)
    e_out, e_lse, _ = _expand_vs_absorb(rng, H=8, T=150, s_q=2, causal=True, dc=512, dr=64, dn=128, dv=128)
    assert e_out <= 1e-10 and e_lse <= 1e-10, (e_out, e_lse)


def test_expand_equals_absorb_handbook_toy(golden):
    """The handbook's own toy sizes, all six tokens new and causal (a prefill), through 4-token pages."""
    g = golden["handbook_toy_example"]
    sh = g["shapes"]
    rng = np.random.default_rng(0)
    e_out, e_lse, _ = _expand_vs_absorb(rng, H=sh["H"], T=sh["T"], s_q=sh["T"], causal=True, dc=sh["DC"],
                                        dr=sh["ROPE"], dn=sh["NOPE"], dv=sh["DV"], page=4)
    assert g["paths_agree"] and e_out < g["paths_agree_atol"]
    assert e_out <= 1e-12 and e_lse <= 1e-12


# ---------------------------------------------------------------- closed forms
def _const_cache(values_per_token, P=2, page=64, D=576):
    cache = np.full((P, page, D), W.BF16_NAN, dtype=np.uint16)
    for t, v in enumerate(values_per_token):
        cache[t // page, t % page, :] = W.f32_to_bf16_bits(np.full(D, v, np.float32))
    return cache


def test_seqlen1_copies_the_latent_exactly():
    rng = np.random.default_rng(3)
    wl = W.make_workload("s1", batch=3, num_heads=16, seqlens=[1, 1, 1], seed=3)
    out, lse = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale)
    for b in range(3):
        c0 = W.bf16_bits_to_f32(wl.cache[wl.block_table[b, 0], 0, :512]).astype(np.float64)
        assert np.array_equal(out[b, 0], np.broadcast_to(c0, (16, 512)))
    assert np.isfinite(lse).all()
    del rng


def test_all_ones_closed_form_pins_scale_and_width():
    """q~ = 1 and token rows all equal a: score = sigma * 576 * a exactly; one token: LSE = score."""
    q = W.f32_to_bf16_bits(np.ones((1, 1, 2, 576), np.float32))
    cache = _const_cache([2.0])
    lse = O.attend(q, cache, np.array([[0, 1]], np.int32), np.array([1], np.int32), softmax_scale=W.SOFTMAX_SCALE)[1]
    assert lse[0, 0, 0] == pytest.approx(float(W.SOFTMAX_SCALE) * 576 * 2.0, rel=1e-15)


def test_seqlen2_closed_form():
    """Two tokens with constant rows a, b: p0 = 1 / (1 + e^(s1 - s0)), LSE = ln(e^s0 + e^s1)."""
    a, b = 0.0625, -0.03125
    q = W.f32_to_bf16_bits(np.ones((1, 1, 1, 576), np.float32))
    cache = _const_cache([a, b])
    out, lse = O.attend(q, cache, np.array([[0, 1]], np.int32), np.array([2], np.int32), softmax_scale=W.SOFTMAX_SCALE)
    s0, s1 = float(W.SOFTMAX_SCALE) * 576 * a, float(W.SOFTMAX_SCALE) * 576 * b
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert out[0, 0, 0] == pytest.approx(np.full(512, p0 * a + (1 - p0) * b), abs=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), abs=1e-14)


@pytest.mark.parametrize("L", [1, 2, 3, 4, 63, 64, 65, 300])
def test_zero_query_gives_mean_and_log_n(L):
    wl = W.make_workload("qz", batch=1, num_heads=4, seqlens=[L], seed=L)
    q = np.zeros_like(wl.q)
    out, lse = O.attend(q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale)
    tok = np.stack([W.bf16_bits_to_f32(wl.cache[wl.block_table[0, t // 64], t % 64, :512]) for t in range(L)])
    assert np.abs(out[0, 0] - tok.astype(np.float64).mean(0)).max() <= 1e-12
    assert np.abs(lse - math.log(L)).max() <= 1e-12


def test_equal_tokens_give_that_token():
    rng = np.random.default_rng(5)
    row = W.f32_to_bf16_bits(rng.standard_normal(576).astype(np.float32))
    L = 100
    cache = np.empty((2, 64, 576), np.uint16)
    cache[:] = row
    q = W.f32_to_bf16_bits(rng.standard_normal((1, 1, 3, 576)).astype(np.float32))
    out, lse = O.attend(q, cache, np.array([[1, 0]], np.int32), np.array([L], np.int32), softmax_scale=W.SOFTMAX_SCALE)
    c = W.bf16_bits_to_f32(row).astype(np.float64)
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    s = float(W.SOFTMAX_SCALE) * (qf[0, 0] @ c)
    assert np.abs(out[0, 0] - c[:512]).max() <= 1e-12
    assert np.abs(lse[0, 0] - (s + math.log(L))).max() <= 1e-12


def test_softmax_weights_sum_to_one():
    """A latent column fixed at 1 for every token reads back sum_t p_t, which must be 1."""
    wl = W.make_workload("sum1", batch=2, num_heads=8, seqlens=[777, 65], seed=9, poison=True)
    for b in range(2):
        for t in range(int(wl.seqlens[b])):
            wl.cache[wl.block_table[b, t // 64], t % 64, 7] = 0x3F80     # 1.0 in bf16
    out, _ = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale)
    assert np.abs(out[..., 7] - 1.0).max() <= 1e-12


# ---------------------------------------------------------------- causal visibility
def test_causal_offsets_follow_pairs_formula(golden):
    """s_q = 2: row 0 sees L-1 keys and row 1 sees L.  A last token that dominates any score it enters
    shows up in row 1 only; and the visible counts add up to q*k - q(q-1)/2."""
    L = 130
    wl = W.make_workload("causal", batch=1, num_heads=2, seqlens=[L], s_q=2, causal=True, seed=21)
    last = wl.block_table[0, (L - 1) // 64], (L - 1) % 64
    wl.cache[last[0], last[1], :] = W.f32_to_bf16_bits(np.full(576, 4.0, np.float32))
    wl.q[:] = W.f32_to_bf16_bits(np.full(wl.q.shape, 1.0, np.float32))
    out, lse = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=True)
    assert np.abs(out[0, 1] - 4.0).max() < 1e-6          # row 1 sees token L-1 and it dominates
    assert abs(out[0, 0].mean() - 4.0) > 1.0             # row 0 does not see it
    q, k = 2, L
    assert (L - 1) + L == q * k - q * (q - 1) // 2


# ---------------------------------------------------------------- split-KV merge
def test_split_merge_equals_unsplit():
    """Windows at random cut points (including 1-token and empty windows) merged by LSE."""
    rng = np.random.default_rng(8)
    seqlens = np.array([2, 3, 200, 517, 64], np.int32)
    wl = W.make_workload("split", batch=5, num_heads=4, seqlens=seqlens, s_q=2, causal=True, seed=8)
    full_o, full_l = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=True)
    J = 4
    cuts = np.zeros((5, J + 1), np.int32)
    for b, L in enumerate(seqlens):
        inner = np.sort(rng.integers(0, L + 1, J - 1))
        if L > 3:
            inner[0] = inner[1]               # force an empty window
        cuts[b] = np.concatenate([[0], inner, [L]])
    parts_o, parts_l = [], []
    for j in range(J):
        o, l = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=True,
                        t_begin=cuts[:, j], t_end=cuts[:, j + 1])
        parts_o.append(o.reshape(-1, 512))
        parts_l.append(l.reshape(-1))
    mo, ml = O.lse_merge(np.stack(parts_o), np.stack(parts_l))
    assert np.abs(mo - full_o.reshape(-1, 512)).max() <= 1e-12
    assert np.abs(ml - full_l.reshape(-1)).max() <= 1e-12


def test_merge_of_empty_parts_is_empty():
    o, l = O.lse_merge(np.zeros((2, 1, 4)), np.full((2, 1), -np.inf))
    assert l[0] == -np.inf and not o.any()


# ---------------------------------------------------------------- stored-input handling
def test_poison_outside_lengths_is_ignored():
    wl = W.make_workload("poison", batch=3, num_heads=4, seqlens=[65, 3, 200], seed=4, spare_pages=5)
    out, lse = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_fp8_cache_is_decoded_times_scale():
    """An FP8 cache gives exactly the result of the same attention over its dequantised bf16-free values:
    compare with a float64 query run over a cache rebuilt from decode(code) * scale at one token."""
    wl = W.make_workload("fp8", batch=1, num_heads=2, seqlens=[1], seed=6, kv_dtype="fp8_e4m3fn")
    out, lse = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale,
                        kv_scale=wl.kv_scale)
    torch = pytest.importorskip("torch")
    pg = wl.block_table[0, 0]
    deq = torch.from_numpy(wl.cache[pg, 0].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * \
        float(wl.kv_scale[pg, 0])
    assert np.array_equal(out[0, 0, 0], deq[:512])        # one token: output is that token's latent


def test_bad_block_table_and_seqlen_are_rejected():
    wl = W.make_workload("bad", batch=1, num_heads=2, seqlens=[10], seed=1)
    bt = wl.block_table.copy()
    bt[0, 0] = wl.num_pages
    with pytest.raises(ValueError, match="block table"):
        O.attend(wl.q, wl.cache, bt, wl.seqlens, softmax_scale=wl.softmax_scale)
    with pytest.raises(ValueError, match="seqlen"):
        O.attend(wl.q, wl.cache, wl.block_table, np.array([65], np.int32), softmax_scale=wl.softmax_scale)


# ------------------------------------------------------------------ expand path pieces used by the prefill
def test_mha_chunks_merged_by_lse_equal_whole():
    """Chunked-prefix attention (the handbook's MHA_CHUNKED_KV reading): attend chunk by chunk and merge
    with the C oracle's LSE merge -- an independent implementation -- gives the unchunked result, also for
    chunks a causal row sees none of (lse -inf, weight 0)."""
    rng = np.random.default_rng(21)
    H, n, L, d = 4, 7, 150, 24
    q = rng.standard_normal((n, H, d))
    k = rng.standard_normal((H, L, d))
    v = rng.standard_normal((H, L, 10))
    qpos, kpos = np.arange(L - n, L), np.arange(L)
    whole_o, whole_l = O.mha_attend(q, k, v, 0.3, qpos, kpos)
    cuts = [0, 40, 41, 97, 146, 148, L]   # the last chunks are partly or wholly after some queries
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = O.mha_attend(q, k[:, a:b], v[:, a:b], 0.3, qpos, kpos[a:b])
        outs.append(o.reshape(n * H, -1))
        lses.append(l.reshape(n * H))
    assert np.isneginf(lses[-1]).sum() == 5 * H     # queries at positions 143-147 see none of [148, 150)
    mo, ml = O.lse_merge(np.stack(outs), np.stack(lses))
    np.testing.assert_allclose(mo, whole_o.reshape(n * H, -1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, whole_l.reshape(n * H), rtol=0, atol=1e-12)


def test_mha_one_key_copies_the_value():
    """With one visible key p = 1, so out = v and lse = scale * (q . k) (closed form)."""
    rng = np.random.default_rng(22)
    q, k, v = rng.standard_normal((1, 3, 8)), rng.standard_normal((3, 1, 8)), rng.standard_normal((3, 1, 5))
    o, l = O.mha_attend(q, k, v, 0.5, np.array([4]), np.array([4]))
    np.testing.assert_array_equal(o[0], v[:, 0])
    np.testing.assert_allclose(l[0], 0.5 * np.einsum("hd,hd->h", q[0], k[:, 0]), rtol=0, atol=1e-14)
    o, l = O.mha_attend(q, k, v, 0.5, np.array([3]), np.array([4]))   # the key is in the future
    assert (o == 0).all() and np.isneginf(l).all()


def test_expand_kv_shapes_and_shared_rope():
    """k = [W_UK[h] c ; k^R] with k^R shared by every head, v = W_UV[h] c (path one of the handbook)."""
    rng = np.random.default_rng(23)
    c, kr = rng.standard_normal((5, 16)), rng.standard_normal((5, 4))
    wuk, wuv = rng.standard_normal((3, 6, 16)), rng.standard_normal((3, 7, 16))
    k, v = O.expand_kv(c, kr, wuk, wuv)
    assert k.shape == (3, 5, 10) and v.shape == (3, 5, 7)
    for h in range(3):
        for t in range(5):
            np.testing.assert_allclose(k[h, t, :6], wuk[h] @ c[t], rtol=0, atol=1e-12)
            np.testing.assert_array_equal(k[h, t, 6:], kr[t])
            np.testing.assert_allclose(v[h, t], wuv[h] @ c[t], rtol=0, atol=1e-12)
