"""bench.py's algorithmic accounting against the figures the pages print (tests/golden/page_figures.json).

The handbook's FLOP script prints per-pair and per-token FLOPs at DeepSeek-V3 shapes and four whole-case totals;
the FlashMLA guide prints 72 MB for batch 8 x context 8192 at 1,152 B per token.  Every function bench.py uses to
turn a workload into FLOPs and bytes is checked against those numbers, so a wrong factor in the reported TFLOP/s
or GB/s fails here."""
import numpy as np
import pytest

import bench


def test_pair_and_token_flops(golden):
    g = golden["handbook_flop_script"]
    H = g["shapes"]["H"]
    assert round(bench.pair_flops_absorb(H) / 1e3) == g["pair_flops_absorb_K"]
    assert round(bench.pair_flops_expand(H) / 1e3) == g["pair_flops_expand_K"]
    assert round(bench.pair_flops_absorb(H) / bench.pair_flops_expand(H), 1) == g["pair_ratio"]
    assert round(bench.expand_flops_per_cached_token(H) / 1e6, 1) == g["expand_flops_per_cached_token_M"]
    assert round(bench.absorb_flops_per_new_token(H) / 1e6, 1) == g["absorb_flops_per_new_token_M"]


@pytest.mark.parametrize("case", range(4))
def test_handbook_case_totals(golden, case):
    """Totals of the four printed cases: new tokens q after k cached (k counts the new ones), causal."""
    g = golden["handbook_flop_script"]
    c = g["cases_GFLOPs"][case]
    H = g["shapes"]["H"]
    pairs = bench.causal_pairs(c["q"], c["k"])
    expand = c["k"] * bench.expand_flops_per_cached_token(H) + pairs * bench.pair_flops_expand(H)
    absorb = c["q"] * bench.absorb_flops_per_new_token(H) + pairs * bench.pair_flops_absorb(H)
    assert round(expand / 1e9, 1) == pytest.approx(c["expand"], abs=0.051)
    assert round(absorb / 1e9, 1) == pytest.approx(c["absorb"], abs=0.051)


def test_crossover_and_intensity(golden):
    g = golden["handbook_flop_script"]
    H = g["shapes"]["H"]
    # new tokens at which the two paths cost the same over a long prefix (k >> q)
    q_star = bench.expand_flops_per_cached_token(H) / (bench.pair_flops_absorb(H) - bench.pair_flops_expand(H))
    assert int(np.ceil(q_star)) == g["crossover_new_tokens"]
    assert round(bench.pair_flops_absorb(H) / bench.kv_bytes_per_token("bf16")) == g["decode_intensity_mla_flop_per_byte"]
    # the handbook's FP8 exercise counts 576 bytes per token (codes only)
    assert round(bench.pair_flops_absorb(H) / (bench.kv_bytes_per_token("fp8_e4m3fn") - 4)) == \
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


@pytest.mark.parametrize("case", ["prefill 8K", "512 tokens after a 32K prefix"])
def test_prefill_counts_are_the_handbooks_path_one_totals(golden, case):
    """bench.py's expand-path FLOPs (expansion of every cached token + causal pairs) reproduce the
    handbook's path-one totals for these shapes."""
    c = next(x for x in golden["handbook_flop_script"]["cases_GFLOPs"] if x["name"] == case)
    assert round(bench.prefill_counts(128, c["q"], c["k"]) / 1e9, 1) == pytest.approx(c["expand"], abs=0.051)
