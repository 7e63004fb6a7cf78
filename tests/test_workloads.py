"""Seeded input generators: determinism, stored formats, and the configured shapes (CPU only)."""
import hashlib

import numpy as np
import pytest

import workloads as W


def _digest(wl):
    h = hashlib.sha256()
    for a in (wl.q, wl.cache, wl.block_table, wl.seqlens) + ((wl.kv_scale,) if wl.kv_scale is not None else ()):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_inputs():
    a = W.make_config("tiny_b1_h16_l256")
    b = W.make_config("tiny_b1_h16_l256")
    assert _digest(a) == _digest(b)
    c = W.make_workload("x", batch=2, num_heads=4, seqlens=[70, 5], seed=1)
    d = W.make_workload("x", batch=2, num_heads=4, seqlens=[70, 5], seed=2)
    assert _digest(c) != _digest(d)


def test_chunked_normal_draw_equals_one_draw():
    r1 = np.random.default_rng(5)
    r2 = np.random.default_rng(5)
    a = W._normal_f32(r1, (37, 3, 11), chunk_rows=4)
    b = r2.standard_normal((37, 3 * 11), dtype=np.float32).reshape(37, 3, 11)
    assert np.array_equal(a, b)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]        # exact ties round to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), ref)


def test_ragged_lengths_for_seed_3():
    rng = np.random.default_rng(3)
    L = W.ragged_seqlens(rng, 128)
    assert (int(L.sum()), int(L.min()), int(np.median(L)), int(L.max())) == (713536, 129, 2446, 28284)
    assert int(((L + 63) // 64).sum()) == 11210


def test_tiny_config_layout():
    wl = W.make_config("tiny_b1_h16_l256")
    assert wl.q.shape == (1, 1, 16, 576) and wl.q.dtype == np.uint16
    assert wl.cache.shape == (4, 64, 576)
    assert np.array_equal(wl.block_table, [[0, 1, 2, 3]])        # identity block table
    assert np.isfinite(W.bf16_bits_to_f32(wl.cache)).all()        # no tail, no spare pages


def test_poison_marks_tail_and_spare_pages():
    wl = W.make_workload("p", batch=2, num_heads=2, seqlens=[65, 10], seed=0, spare_pages=2)
    vals = W.bf16_bits_to_f32(wl.cache)
    referenced = set(wl.block_table[wl.block_table >= 0].tolist())
    for p in range(wl.num_pages):
        if p not in referenced:
            assert np.isnan(vals[p]).all()
    last0 = wl.block_table[0, 1]
    assert np.isfinite(vals[last0, :1]).all() and np.isnan(vals[last0, 1:]).all()
    assert (wl.block_table[1, 1:] == -1).all()


def test_fp8_quantisation_uses_per_token_amax():
    torch = pytest.importorskip("torch")
    wl = W.make_workload("f", batch=1, num_heads=2, seqlens=[64], seed=3, kv_dtype="fp8_e4m3fn", permute_pages=False)
    deq = torch.from_numpy(wl.cache).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.abs(deq).max(axis=-1).max() == 448.0               # every token hits the top code
    assert (np.abs(deq).max(axis=-1) == 448.0).all()
    assert wl.kv_scale.dtype == np.float32 and (wl.kv_scale > 0).all()
