"""bench.py's algorithmic accounting against the figures the pages print (tests/golden/page_figures.json).

bench.py counts FLOPs and bytes from the contractions the kernels perform (a 576-wide score and a 512-wide
weighted row per head and visible key on the absorb path; the expansion products and a 192/128-wide attention on
the expand path).  The handbook's FLOP script prints per-pair and per-token FLOPs at DeepSeek-V3 shapes and four
whole-case totals; the FlashMLA guide prints 72 MB for batch 8 x context 8192 at 1,152 B per token.  Every
function bench.py uses to turn a workload into FLOPs and bytes is checked against those numbers, so a wrong
factor in the reported TFLOP/s or GB/s fails here."""
import numpy as np
import pytest

import bench
import workloads as W
from oracle import oracle as O


def test_pair_and_token_flops(golden):
    g = golden["handbook_flop_script"]
    H = g["shapes"]["H"]
    assert round(bench.decode_flops_per_key(H) / 1e3) == g["pair_flops_absorb_K"]
    assert round(bench.mha_flops_per_key(H) / 1e3) == g["pair_flops_expand_K"]
    assert round(bench.decode_flops_per_key(H) / bench.mha_flops_per_key(H), 1) == g["pair_ratio"]
    assert round(bench.expansion_flops_per_token(H) / 1e6, 1) == g["expand_flops_per_cached_token_M"]
    assert round(bench.projection_flops_per_token(H) / 1e6, 1) == g["absorb_flops_per_new_token_M"]


@pytest.mark.parametrize("case", range(4))
def test_handbook_case_totals(golden, case):
    """Totals of the four printed cases: q new tokens at the end of k tokens (k counts them), causal."""
    g = golden["handbook_flop_script"]
    c = g["cases_GFLOPs"][case]
    H = g["shapes"]["H"]
    keys = sum(bench.visible_keys(c["k"], c["q"], True))
    expand = c["k"] * bench.expansion_flops_per_token(H) + keys * bench.mha_flops_per_key(H)
    absorb = c["q"] * bench.projection_flops_per_token(H) + keys * bench.decode_flops_per_key(H)
    assert round(expand / 1e9, 1) == pytest.approx(c["expand"], abs=0.051)
    assert round(absorb / 1e9, 1) == pytest.approx(c["absorb"], abs=0.051)


def test_crossover_and_intensity(golden):
    g = golden["handbook_flop_script"]
    H = g["shapes"]["H"]
    # new tokens at which the two paths cost the same over a long prefix (k >> q)
    q_star = bench.expansion_flops_per_token(H) / (bench.decode_flops_per_key(H) - bench.mha_flops_per_key(H))
    assert int(np.ceil(q_star)) == g["crossover_new_tokens"]
    assert round(bench.decode_flops_per_key(H) / bench.kv_bytes_per_token("bf16")) == \
        g["decode_intensity_mla_flop_per_byte"]
    # the handbook's FP8 exercise counts 576 bytes per token (codes only)
    assert round(bench.decode_flops_per_key(H) / (bench.kv_bytes_per_token("fp8_e4m3fn") - 4)) == \
        golden["handbook_fp8_exercise"]["fp8_intensity_flop_per_byte"]


def test_guide_cache_size(golden):
    g = golden["flashmla_guide_simulation"]
    assert bench.kv_bytes_per_token("bf16") == g["bytes_per_token"]
    seqlens = np.full(g["batch"], g["context"])
    _, kv, _ = bench.workload_counts(seqlens, 128, 1, False)
    assert round(kv / 2**20) == g["mla_MB"]


def test_headline_and_mtp_counts():
    """The configurations' own totals (closed forms): B=64 x 4096 tokens; B=32 x 8192 with two causal new tokens."""
    f, kv, total = bench.workload_counts(np.full(64, 4096), 128, 1, False)
    assert f == 64 * 4096 * 278528 and kv == 64 * 4096 * 1152
    assert total == kv + 64 * 128 * (576 * 2 + 512 * 2 + 4) + 64 * 4 + 64 * 64 * 4
    f2, _, _ = bench.workload_counts(np.full(32, 8192), 128, 2, True)
    assert f2 == 32 * (2 * 8192 - 1) * 278528


def test_visible_keys_are_the_oracles_causal_rule():
    """The accounting's visible-key count equals the keys the oracle attends to: a row whose query is zero
    averages exactly its visible keys, so a latent column holding the token index reads back their mean."""
    L, s_q = 70, 3
    wl = W.make_workload("vk", batch=1, num_heads=1, seqlens=[L], s_q=s_q, causal=True, seed=2, poison=False)
    q = np.zeros_like(wl.q)
    cache = wl.cache.copy()
    for t in range(L):
        cache[wl.block_table[0, t // 64], t % 64, 0] = W.f32_to_bf16_bits(np.float32([t]))[0]
    out, lse = O.attend(q, cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=True)
    for i, n in enumerate(bench.visible_keys(L, s_q, True)):
        assert out[0, i, 0, 0] == pytest.approx((n - 1) / 2, abs=1e-12)
        assert lse[0, i, 0] == pytest.approx(np.log(n), abs=1e-12)


@pytest.mark.parametrize("case", ["prefill 8K", "512 tokens after a 32K prefix"])
def test_prefill_counts_are_the_handbooks_path_one_totals(golden, case):
    """bench.py's expand-path FLOPs (expansion of every cached token + causal pairs) reproduce the
    handbook's path-one totals for these shapes."""
    c = next(x for x in golden["handbook_flop_script"]["cases_GFLOPs"] if x["name"] == case)
    assert round(bench.prefill_counts(128, c["q"], c["k"]) / 1e9, 1) == pytest.approx(c["expand"], abs=0.051)


# ------------------------------------------------------------------ cache-size figures the handbook prints
def test_cache_is_576_numbers_per_token_per_layer(golden):
    """The handbook's latent cache: 576 numbers per token per layer.  The stored cache row, the query width the
    library and the oracle read, and bench.py's byte count all have that width."""
    import mla_latent_kv_fwd_amd as M
    g = golden["handbook_cache"]
    n = g["numbers_per_token_per_layer"]
    assert W.D_QK == n and M.HEAD_DIM_QK == n and bench.D_QK == n
    wl = W.make_workload("w", batch=1, num_heads=2, seqlens=[3], seed=0)
    assert wl.cache.shape[-1] == n and wl.q.shape[-1] == n
    assert bench.kv_bytes_per_token("bf16") == 2 * n
    # over the model's layers in bf16: the handbook's ~70 KB per token
    assert round(g["layers"] * n * 2 / 1000) == g["bf16_KB_over_layers"]


def test_mha_cache_comparison(golden):
    """The handbook's MHA cache for comparison: K and V of 128 heads x 128 dims per token per layer."""
    g = golden["handbook_cache"]
    H = golden["handbook_flop_script"]["shapes"]["H"]
    assert 2 * H * bench.D_V == g["mha_numbers_per_token_per_layer"]
    assert g["mha_numbers_per_token_per_layer"] / g["numbers_per_token_per_layer"] > 56


def test_toy_example_numbers_per_token(golden):
    """The handbook's toy example: its expand path keeps H (NOPE + ROPE) key numbers and H DV value numbers per
    token (80), the absorb path DC + ROPE latent numbers (20).  Counted from the oracle's own tensors at the toy's
    shapes: the expanded k and v of one token, and one cache row."""
    t = golden["handbook_toy_example"]
    s = t["shapes"]
    rng = np.random.default_rng(0)
    lat = rng.standard_normal((1, s["DC"]))
    rope = rng.standard_normal((1, s["ROPE"]))
    w_uk = rng.standard_normal((s["H"], s["NOPE"], s["DC"]))
    w_uv = rng.standard_normal((s["H"], s["DV"], s["DC"]))
    k, v = O.expand_kv(lat, rope, w_uk, w_uv)
    assert k[:, 0].size + v[:, 0].size == t["mha_numbers_per_token"]
    assert lat.shape[1] + rope.shape[1] == t["mla_numbers_per_token"]
