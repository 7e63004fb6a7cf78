"""Seeded synthetic inputs for MLA absorb-path decode.

This module only draws inputs: random numbers, rounding to the stored formats,
block tables and NaN poison.  It contains none of the attention arithmetic, and
both the HIP path's tests/benchmark and the fp64 oracle read what it produces.

Shapes follow DeepSeek-V3's MLA (128 heads, a 512-wide latent plus a 64-wide
RoPE key per cached token, so 576 numbers per token; pages of 64 tokens), as
the handbook page "MLA inference: two computation paths and FlashMLA" gives
them in "Which is faster" and in its FlashMLA paragraph.

Recipe (fixed so any run can be reproduced):
  * RNG: numpy ``default_rng(seed)`` (PCG64); draw order on it: seqlens
    (ragged only) -> page permutation -> one 63-bit root seed for the values.
  * The values come from PCG64 streams spawned from that root
    (``SeedSequence(root).spawn``): stream b draws request b's queries
    [s_q, H, 576]; stream B + j draws the latent [n, 64, 512] and then the RoPE
    part [n, 64, 64] of pages 64 j .. 64 j + n - 1 (physical page order).  The
    streams are independent, so blocks are drawn on several threads at once and
    encoded straight into the stored format (no whole-cache float32 copy).
  * Values are drawn in float32 and stored as bf16 with round-to-nearest-even;
    the FP8 cache stores OCP E4M3FN codes of x / s_t with a per-token scale
    s_t = amax_t / 448 over all 576 numbers of the token (1 when amax is 0).
  * Cache rows beyond a request's length in its last page, and every page no
    request references, are filled with NaN: results must not depend on them.
  * Block-table entries past a request's last page are -1.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE
PAGE = 64
SOFTMAX_SCALE = np.float32(1.0 / math.sqrt(128 + 64))   # 1/sqrt(d_nope + d_rope)

BF16_NAN = np.uint16(0x7FC0)
E4M3FN_NAN = np.uint8(0x7F)
E4M3FN_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Encode float32 to OCP E4M3FN codes, round-to-nearest-even, saturating at +-448.

    Uses PyTorch's float8_e4m3fn cast on values already clipped to the finite range.
    """
    import torch
    clipped = np.clip(np.asarray(x, dtype=np.float32), -E4M3FN_MAX, E4M3FN_MAX)
    return torch.from_numpy(np.ascontiguousarray(clipped)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclasses.dataclass
class Workload:
    name: str
    q: np.ndarray               # uint16 bf16 bits [B, s_q, H, 576]
    cache: np.ndarray           # uint16 bf16 bits or uint8 E4M3FN codes [P, 64, 576]
    kv_scale: Optional[np.ndarray]  # float32 [P, 64] (FP8 only)
    block_table: np.ndarray     # int32 [B, max_blocks]
    seqlens: np.ndarray         # int32 [B]
    s_q: int
    num_heads: int
    causal: bool
    softmax_scale: np.float32 = SOFTMAX_SCALE

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.cache.shape[0])

    @property
    def kv_dtype(self) -> str:
        return "fp8_e4m3fn" if self.cache.dtype == np.uint8 else "bf16"


def _normal_f32(rng: np.random.Generator, shape, chunk_rows: int = 1 << 20) -> np.ndarray:
    """standard_normal in float32, drawn in row chunks (same stream as one draw) to bound memory."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
    return out


PAGES_PER_STREAM = 64   # pages drawn from one spawned value stream
_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _parallel(fn, n):
    """fn(i) for i < n on a thread pool (numpy's fills and ufuncs release the GIL)."""
    if n <= 1 or _WORKERS == 1:
        for i in range(n):
            fn(i)
        return
    with concurrent.futures.ThreadPoolExecutor(_WORKERS) as ex:
        for f in [ex.submit(fn, i) for i in range(n)]:
            f.result()


def _encode_fp8_tokens(x: np.ndarray):
    """Per-token scale s = amax / 448 over the last axis (1 when amax is 0) and the E4M3FN codes of x / s."""
    amax = np.abs(x).max(axis=-1)
    s = np.where(amax > 0, amax / np.float32(E4M3FN_MAX), np.float32(1.0)).astype(np.float32)
    return f32_to_e4m3fn(x / s[..., None]), s


def make_workload(name: str, *, batch: int, num_heads: int, seqlens: Sequence[int] | np.ndarray, s_q: int = 1,
                  causal: bool = False, seed: int = 0, latent_std: float = 1.0, q_std: float = 1.0,
                  rope_std: float = 1.0, kv_dtype: str = "bf16", permute_pages: bool = True,
                  spare_pages: int = 0, max_blocks: Optional[int] = None, poison: bool = True,
                  rng: Optional[np.random.Generator] = None, shape_values=None) -> Workload:
    """Draw one decode batch.  ``seqlens`` counts the new tokens (each >= s_q).

    ``shape_values(q, latent, rope, block_table, seqlens, rng)``, if given, may
    rewrite the float32 draws in place before they are encoded (structured
    inputs for a test; the whole cache is then held in float32 once).
    """
    if kv_dtype not in ("bf16", "fp8_e4m3fn"):
        raise ValueError(kv_dtype)
    rng = np.random.default_rng(seed) if rng is None else rng
    seqlens = np.asarray(seqlens, dtype=np.int32)
    assert seqlens.shape == (batch,) and (seqlens >= s_q).all()
    npages = (seqlens.astype(np.int64) + PAGE - 1) // PAGE
    used = int(npages.sum())
    P = used + spare_pages
    mb = int(npages.max()) if max_blocks is None else max_blocks
    assert mb >= npages.max()

    perm = rng.permutation(P).astype(np.int32) if permute_pages else np.arange(P, dtype=np.int32)
    block_table = np.full((batch, mb), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        block_table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])

    nblk = (P + PAGES_PER_STREAM - 1) // PAGES_PER_STREAM
    streams = np.random.SeedSequence(int(rng.integers(0, 1 << 63))).spawn(batch + nblk)
    gen = lambda i: np.random.Generator(np.random.PCG64(streams[i]))

    q_bits = np.empty((batch, s_q, num_heads, D_QK), dtype=np.uint16)
    q32 = np.empty((batch, s_q, num_heads, D_QK), dtype=np.float32) if shape_values is not None else None

    def draw_q(b):
        x = gen(b).standard_normal((s_q, num_heads, D_QK), dtype=np.float32)
        if q_std != 1.0:
            x *= np.float32(q_std)
        if q32 is not None:
            q32[b] = x
        else:
            q_bits[b] = f32_to_bf16_bits(x)

    def draw_pages(j):
        p0 = j * PAGES_PER_STREAM
        n = min(P, p0 + PAGES_PER_STREAM) - p0
        g = gen(batch + j)
        lat = g.standard_normal((n, PAGE, D_LATENT), dtype=np.float32)
        rope = g.standard_normal((n, PAGE, D_ROPE), dtype=np.float32)
        if latent_std != 1.0:
            lat *= np.float32(latent_std)
        if rope_std != 1.0:
            rope *= np.float32(rope_std)
        return p0, n, lat, rope

    kv_scale = np.empty((P, PAGE), dtype=np.float32) if kv_dtype == "fp8_e4m3fn" else None
    cache = np.empty((P, PAGE, D_QK), dtype=np.uint16 if kv_dtype == "bf16" else np.uint8)

    def encode(p0, n, lat, rope):
        if kv_dtype == "bf16":
            cache[p0:p0 + n, :, :D_LATENT] = f32_to_bf16_bits(lat)
            cache[p0:p0 + n, :, D_LATENT:] = f32_to_bf16_bits(rope)
        else:
            cache[p0:p0 + n], kv_scale[p0:p0 + n] = _encode_fp8_tokens(np.concatenate([lat, rope], axis=-1))

    if shape_values is None:
        _parallel(draw_q, batch)
        _parallel(lambda j: encode(*draw_pages(j)), nblk)
    else:
        latent = np.empty((P, PAGE, D_LATENT), dtype=np.float32)
        rope_all = np.empty((P, PAGE, D_ROPE), dtype=np.float32)

        def fill(j):
            p0, n, lat, rope = draw_pages(j)
            latent[p0:p0 + n] = lat
            rope_all[p0:p0 + n] = rope

        _parallel(draw_q, batch)
        _parallel(fill, nblk)
        shape_values(q32, latent, rope_all, block_table, seqlens, rng)
        q_bits[...] = f32_to_bf16_bits(q32)
        _parallel(lambda j: encode(j * PAGES_PER_STREAM, min(P, (j + 1) * PAGES_PER_STREAM) - j * PAGES_PER_STREAM,
                                   latent[j * PAGES_PER_STREAM:(j + 1) * PAGES_PER_STREAM],
                                   rope_all[j * PAGES_PER_STREAM:(j + 1) * PAGES_PER_STREAM]), nblk)
        del latent, rope_all, q32

    if poison:
        nan = BF16_NAN if kv_dtype == "bf16" else E4M3FN_NAN
        referenced = np.zeros(P, dtype=bool)
        for b in range(batch):
            referenced[block_table[b, :npages[b]]] = True
            tail = int(seqlens[b]) % PAGE
            if tail:
                last = block_table[b, npages[b] - 1]
                cache[last, tail:] = nan
                if kv_scale is not None:
                    kv_scale[last, tail:] = np.nan
        cache[~referenced] = nan
        if kv_scale is not None:
            kv_scale[~referenced] = np.nan
    return Workload(name=name, q=q_bits, cache=cache, kv_scale=kv_scale, block_table=block_table, seqlens=seqlens,
                    s_q=s_q, num_heads=num_heads, causal=causal)


def make_score_jump_workload(name: str, *, seqlens: Sequence[int], jumps: Sequence[Sequence[tuple]],
                             num_heads: int = 128, kv_dtype: str = "bf16", seed: int = 0,
                             rope_high: float = 0.7) -> Workload:
    """A batch whose scores jump: most keys give every head a score near 0, and a
    few tokens per request (``jumps[b]`` = list of (first, count, level)) score
    about 6.5 * level nats higher (a RoPE-part key of rope_high * level against a
    query RoPE part of 2).  Low and high tokens carry latents with different
    dim-dependent means, so each group's share of the softmax shows in the output.
    """
    def shape(q, latent, rope, block_table, sl, rng):
        q[..., :D_LATENT] *= np.float32(0.05)
        q[..., D_LATENT:] = np.float32(2.0) + np.float32(0.05) * q[..., D_LATENT:]
        dims = np.arange(D_LATENT, dtype=np.float32)
        low_mean = np.sin(np.float32(0.05) * dims).astype(np.float32)
        high_mean = -np.cos(np.float32(0.11) * dims).astype(np.float32)
        latent *= np.float32(0.3)
        latent += low_mean
        rope *= np.float32(0.05)
        for b, spans in enumerate(jumps):
            for first, count, level in spans:
                for t in range(first, first + count):
                    assert t < sl[b]
                    page, slot = block_table[b, t // PAGE], t % PAGE
                    latent[page, slot] += high_mean - low_mean
                    rope[page, slot] += np.float32(rope_high * level)

    return make_workload(name, batch=len(seqlens), num_heads=num_heads, seqlens=seqlens, seed=seed,
                         kv_dtype=kv_dtype, spare_pages=2, shape_values=shape)


def ragged_seqlens(rng: np.random.Generator, batch: int, lo: int = 128, hi: int = 32768) -> np.ndarray:
    """Per-request lengths drawn log-uniform in [lo, hi]."""
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), batch))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


# The five measured/parity configurations (descriptions are the workload names used everywhere).
CONFIGS = {
    "tiny_b1_h16_l256": dict(batch=1, num_heads=16, seqlen=256, seed=1, permute_pages=False),
    "dsv3_b64_h128_l4096": dict(batch=64, num_heads=128, seqlen=4096, seed=2, latent_std=0.5),
    "ragged_b128_h128_l128_32768": dict(batch=128, num_heads=128, seqlen="ragged", seed=3),
    "mtp_b32_h128_sq2_l8192": dict(batch=32, num_heads=128, seqlen=8192, seed=4, s_q=2, causal=True),
    "fp8_b128_h128_l16384": dict(batch=128, num_heads=128, seqlen=16384, seed=5, kv_dtype="fp8_e4m3fn"),
}
HEADLINE = "dsv3_b64_h128_l4096"


def make_config(name: str, **overrides) -> Workload:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = cfg.pop("seed")
    rng = np.random.default_rng(seed)
    seqlen = cfg.pop("seqlen")
    batch = cfg["batch"]
    if seqlen == "ragged":
        seqlens = ragged_seqlens(rng, batch)
    else:
        seqlens = np.full(batch, seqlen, dtype=np.int32)
    return make_workload(name, seqlens=seqlens, rng=rng, **cfg)


D_NOPE = 128
D_V = 128


@dataclasses.dataclass
class ProjInputs:
    q_nope: np.ndarray   # uint16 bf16 bits [T, H, 128]
    q_rope: np.ndarray   # uint16 bf16 bits [T, H, 64]
    w_uk: np.ndarray     # uint16 bf16 bits [H, 128, 512]   (k^N = W_UK[h] c)
    w_uv: np.ndarray     # uint16 bf16 bits [H, 128, 512]   (v = W_UV[h] c)


def make_proj_inputs(*, tokens: int, num_heads: int, seed: int = 0) -> ProjInputs:
    """Per-head query parts and up-projection weights, bf16 bits.

    q^N and q^R are standard normal; the weights are normal with std
    1/sqrt(fan-in) (W_UK: 128, so an absorbed query number has variance ~1 like
    the decode workloads' q; W_UV: 512).
    """
    rng = np.random.default_rng(seed)
    q_nope = rng.standard_normal((tokens, num_heads, D_NOPE), dtype=np.float32)
    q_rope = rng.standard_normal((tokens, num_heads, D_ROPE), dtype=np.float32)
    w_uk = rng.standard_normal((num_heads, D_NOPE, D_LATENT), dtype=np.float32) * np.float32(1 / math.sqrt(D_NOPE))
    w_uv = rng.standard_normal((num_heads, D_V, D_LATENT), dtype=np.float32) * np.float32(1 / math.sqrt(D_LATENT))
    return ProjInputs(q_nope=f32_to_bf16_bits(q_nope), q_rope=f32_to_bf16_bits(q_rope), w_uk=f32_to_bf16_bits(w_uk),
                      w_uv=f32_to_bf16_bits(w_uv))


@dataclasses.dataclass
class PrefillWorkload:
    name: str
    q: np.ndarray             # uint16 bf16 bits [n, H, 192]  ([q^N ; q^R])
    cache: np.ndarray         # uint16 bf16 bits [P, 64, 576]  (the request's latents, prefix and new tokens)
    block_table: np.ndarray   # int32 [max_blocks]  (the request's row)
    w_uk: np.ndarray          # uint16 bf16 bits [H, 128, 512]
    w_uv: np.ndarray          # uint16 bf16 bits [H, 128, 512]
    seqlen: int               # L: tokens in the cache (prefix + new)
    num_new: int              # n: new tokens, the last n positions
    num_heads: int
    softmax_scale: np.float32 = SOFTMAX_SCALE

    @property
    def num_pages(self) -> int:
        return int(self.cache.shape[0])


def make_prefill_workload(name: str, *, num_heads: int, num_new: int, seqlen: int, seed: int = 0,
                          spare_pages: int = 2, poison: bool = True) -> PrefillWorkload:
    """One request for the expand path: its L cached tokens (permuted pages, NaN past its end and in
    spare pages, as for decode), queries q = [q^N ; q^R] ~ N(0, 1) for the last n positions, and
    W_UK, W_UV ~ N(0, 1/512) so that k^N = W_UK c and v = W_UV c have the latent's variance."""
    assert 1 <= num_new <= seqlen
    wl = make_workload(name, batch=1, num_heads=1, seqlens=[seqlen], seed=seed, spare_pages=spare_pages,
                       poison=poison)
    rng = np.random.default_rng(seed + 7919)
    q = rng.standard_normal((num_new, num_heads, D_NOPE + D_ROPE), dtype=np.float32)
    w_uk = rng.standard_normal((num_heads, D_NOPE, D_LATENT), dtype=np.float32) * np.float32(1 / math.sqrt(D_LATENT))
    w_uv = rng.standard_normal((num_heads, D_V, D_LATENT), dtype=np.float32) * np.float32(1 / math.sqrt(D_LATENT))
    return PrefillWorkload(name=name, q=f32_to_bf16_bits(q), cache=wl.cache, block_table=wl.block_table[0].copy(),
                           w_uk=f32_to_bf16_bits(w_uk), w_uv=f32_to_bf16_bits(w_uv), seqlen=seqlen,
                           num_new=num_new, num_heads=num_heads)


def prefill_latents(pw: PrefillWorkload) -> tuple[np.ndarray, np.ndarray]:
    """The request's latent c [L, 512] and RoPE key k^R [L, 64] as float32, gathered through its block table."""
    L = pw.seqlen
    rows = pw.cache[pw.block_table[:(L + PAGE - 1) // PAGE]].reshape(-1, D_QK)[:L]
    x = bf16_bits_to_f32(rows)
    return x[:, :D_LATENT], x[:, D_LATENT:]
