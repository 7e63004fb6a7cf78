#!/usr/bin/env python3
"""Benchmark of one MLA absorb-path decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--copies C] [--no-cpu]

A step is the whole hot path over one batch of synthetic inputs already
resident in HBM: the split plan, the attention kernel over the paged cache and
the LSE combine.  The timed region holds exactly K steps between device
synchronisations.  The cache is cycled over C independent copies so repeats
cannot be served from the 256 MB last-level cache (C is chosen so the copies
total at least twice that, unless given).

Prints one JSON line.  ``value`` is algorithmic TFLOP/s of the whole step;
``projections`` times the two per-head projections on either side of the step
(W_UK absorbed into the query, W_UV on the latent output) separately, and
``prefill`` the chunked expand path on 512 new tokens after a 32K prefix (or,
with ``--prefill prefill_h128_n8192``, a prefill of 8K new tokens);
``roofline`` describes the attention kernel alone (its launches are timed with
HIP events on the stream it runs on, inside the timed region, on every 10th
step; the plan and combine are timed in a separate pass because each event pair
costs GPU time); ``cpu_baseline`` is the fp64 oracle run on a bounded sample of
the same workload's rows on the host cores.  Every timed leg starts after the
GPU has been kept busy for a while, so that its clocks have left the idle state.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense bf16
MALL_BYTES = 256 << 20            # last-level (Infinity) cache
D_LATENT, D_ROPE, D_NOPE, D_V = 512, 64, 128, 128


# ---------------------------------------------------------------- algorithmic accounting
def pair_flops_absorb(H, dc=D_LATENT, dr=D_ROPE):
    """FLOPs per (query token, cached token) pair on the absorb path: a (dc+dr)-wide score and a
    dc-wide weighted sum for each of H heads (handbook FLOP script)."""
    return 2 * H * (dc + dr) + 2 * H * dc


def pair_flops_expand(H, dn=D_NOPE, dr=D_ROPE, dv=D_V):
    return 2 * H * (dn + dr) + 2 * H * dv


def expand_flops_per_cached_token(H, dc=D_LATENT, dn=D_NOPE, dv=D_V):
    return 2 * dc * H * (dn + dv)


def absorb_flops_per_new_token(H, dc=D_LATENT, dn=D_NOPE, dv=D_V):
    return 2 * H * dn * dc + 2 * H * dc * dv


def causal_pairs(q, k):
    """(query, key) pairs when q new tokens follow and are counted in k tokens, causal among the new ones."""
    return q * k - q * (q - 1) // 2


def kv_bytes_per_token(dtype="bf16", dc=D_LATENT, dr=D_ROPE):
    """Cache bytes read per cached token: 2 bytes per number in bf16; 1 per number plus a 4-byte scale in FP8."""
    return (dc + dr) * 2 if dtype == "bf16" else (dc + dr) + 4


def workload_counts(seqlens, H, s_q, causal, kv_dtype="bf16"):
    """(FLOPs, KV bytes, total algorithmic bytes) of one decode step over these requests."""
    pairs = 0
    for L in seqlens:
        pairs += causal_pairs(s_q, int(L)) if causal else s_q * int(L)
    flops = pairs * pair_flops_absorb(H)
    kv = sum(int(L) for L in seqlens) * kv_bytes_per_token(kv_dtype)
    B = len(seqlens)
    io = B * s_q * H * (D_LATENT + D_ROPE) * 2 + B * s_q * H * D_LATENT * 2 + B * s_q * H * 4
    tables = B * 4 + sum(-(-int(L) // 64) for L in seqlens) * 4
    return flops, kv, kv + io + tables


# ---------------------------------------------------------------- benchmark
def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None)
    ap.add_argument("--copies", type=int, default=0, help="independent cache copies to cycle (0 = auto)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record the attention kernel's event pair on every Nth timed step")
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="keep the GPU busy this long after the W warm-up steps (0 for counter runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the CPU baseline sample")
    ap.add_argument("--no-proj", action="store_true", help="skip the projection kernels' measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the expand-path (prefill) measurement")
    ap.add_argument("--prefill", default="extend_h128_p32768_n512", choices=sorted(PREFILL_WORKLOADS),
                    help="expand-path workload to measure")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB -> 1 GiB elementwise copy (calibrates the HBM byte counters)")
    return ap.parse_args()


COPY_PROBE_BYTES = 1 << 30
# Sustained work before any timed region: the GPU's clocks ramp up over the first
# milliseconds of a burst that starts from idle (measured at the headline shape:
# ~120 us per step over the first 40 steps after 0.5 s idle, 98-99 us sustained),
# so a timed region entered from idle clocks would time the ramp, not the kernels.
WARM_SECONDS = 0.25


def keep_busy(torch, fn, seconds=WARM_SECONDS, min_calls=1):
    """Untimed calls fn(i) until the GPU has run them for `seconds` (host and device kept within 64 calls
    of each other by periodic synchronisation); returns the number of calls."""
    calls = 0
    t0 = time.perf_counter()
    while calls < min_calls or time.perf_counter() - t0 < seconds:
        fn(calls)
        calls += 1
        if calls % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return calls


def copy_probe():
    """Five launches of a plain elementwise kernel that reads 1 GiB and writes 1 GiB (fp32 negation):
    the reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE readings to bytes."""
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES, "copy_probe_bytes_written": COPY_PROBE_BYTES,
                      "launches": 5}))
    return 0


def kernel_source_digest():
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_kv_fwd_amd", "csrc",
                        "mla_decode_kernel.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload, kv_dtype):
    """HBM bytes per attention-kernel launch from the committed counter summary of this workload, or None
    when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip().strip("`")] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return int(fields["decode_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def projection_bytes(T, H):
    """Algorithmic HBM bytes of one launch of each projection: weights, inputs and outputs once."""
    w = H * D_NOPE * D_LATENT * 2
    absorb = w + T * H * (D_NOPE + D_ROPE) * 2 + T * H * (D_LATENT + D_ROPE) * 2
    project = w + T * H * D_LATENT * 2 + T * H * D_V * 2
    return absorb, project


def bench_projections(torch, M, W, T, H, launches=200):
    """The two projections around the attention (W_UK absorbed into the query, W_UV on the latent output)
    at this step's T = batch * s_q query rows: average time per launch over back-to-back launches between
    one event pair, with weights, inputs and outputs cycled over copies that together exceed twice the
    last-level cache."""
    import numpy as np
    b_abs, b_proj = projection_bytes(T, H)
    nsets = max(2, math.ceil(2 * MALL_BYTES / (b_abs + b_proj)))
    rng = np.random.default_rng(11)
    pi = W.make_proj_inputs(tokens=T, num_heads=H, seed=10)
    o_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H, D_LATENT), dtype=np.float32) * np.float32(0.3))
    dev = lambda b: torch.from_numpy(b.view(np.int16)).to("cuda")
    base = [dev(pi.q_nope), dev(pi.q_rope), dev(pi.w_uk), dev(pi.w_uv), dev(o_bits)]
    sets = []
    for _ in range(nsets):
        qn, qr, wuk, wuv, o = (x.clone() for x in base)
        sets.append((qn, qr, wuk, wuv, o, torch.empty((T, H, D_LATENT + D_ROPE), dtype=torch.int16, device="cuda"),
                     torch.empty((T, H, D_V), dtype=torch.int16, device="cuda")))
    calls = {"absorb": lambda z: M.absorb_q(z[0], z[1], z[2], out=z[5]),
             "project": lambda z: M.project_out(z[4], z[3], out=z[6])}
    res = {}
    for name, fn in calls.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        keep_busy(torch, lambda i: fn(sets[i % nsets]), seconds=0.1, min_calls=2 * nsets)
        e0.record()
        for i in range(launches):
            fn(sets[i % nsets])
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / launches
    gbps = lambda nbytes, us: nbytes / (us * 1e-6) / 1e9
    return {"tokens": T, "heads": H,
            "absorb_q": {"us": round(res["absorb"], 3), "bytes": b_abs, "gbps": round(gbps(b_abs, res["absorb"]), 1),
                         "frac_hbm": round(gbps(b_abs, res["absorb"]) / HBM_PEAK_GBPS, 4)},
            "project_out": {"us": round(res["project"], 3), "bytes": b_proj,
                            "gbps": round(gbps(b_proj, res["project"]), 1),
                            "frac_hbm": round(gbps(b_proj, res["project"]) / HBM_PEAK_GBPS, 4)},
            "timing": f"{launches} back-to-back launches between one event pair, {nsets} input/weight copies, "
                      "after the timed region; not part of the step"}


# The handbook's two expand-path shapes: 512 new tokens after a 32K prefix, and a prefill of 8K new tokens.
PREFILL_WORKLOADS = {
    "extend_h128_p32768_n512": dict(num_heads=128, num_new=512, seqlen=32768 + 512, chunk_tokens=8192),
    "prefill_h128_n8192": dict(num_heads=128, num_new=8192, seqlen=8192, chunk_tokens=8192),
}


def prefill_counts(H, n, L):
    """Algorithmic FLOPs of the expand path for n new tokens after L - n cached ones: expanding every one of
    the L cached tokens into K and V for H heads, plus the causal (query, key) pairs at 2H(192 + 128) each
    (the handbook's path-one accounting)."""
    return L * expand_flops_per_cached_token(H) + causal_pairs(n, L) * pair_flops_expand(H)


def bench_prefill(torch, M, W, name, launches=10):
    """The chunked expand path (mla_chunked_prefill) on one of the handbook's shapes: average time per call
    over back-to-back calls between one event pair, after the timed region."""
    import numpy as np
    cfg = PREFILL_WORKLOADS[name]
    H, n, L = cfg["num_heads"], cfg["num_new"], cfg["seqlen"]
    pw = W.make_prefill_workload(name, num_heads=H, num_new=n, seqlen=L, seed=1, poison=False)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
    q, kv, bt, wuk, wuv = dev(pw.q), dev(pw.cache), dev(pw.block_table), dev(pw.w_uk), dev(pw.w_uv)
    pre = M.MlaPrefill(num_heads=H, num_new=n, seqlen=L, num_pages=pw.num_pages, max_blocks=len(pw.block_table),
                       chunk_tokens=cfg["chunk_tokens"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    keep_busy(torch, lambda i: pre(q, kv, bt, wuk, wuv), seconds=0.1, min_calls=3)
    e0.record()
    for _ in range(launches):
        pre(q, kv, bt, wuk, wuv)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    flops = prefill_counts(H, n, L)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": name, "heads": H, "new_tokens": n, "seqlen": L, "chunk_tokens": cfg["chunk_tokens"],
            "ms": round(ms, 4), "gflop": round(flops / 1e9, 1), "tflops": round(tflops, 1),
            "frac_mfma": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "timing": f"{launches} back-to-back calls between one event pair, after the timed region; "
                      "not part of the step"}


def cpu_baseline(wl, target_s):
    """fp64 oracle on a bounded sample of rows; returns the dict for the JSON line."""
    import numpy as np
    from oracle import oracle as O
    total = wl.batch * wl.s_q * wl.num_heads
    rng = np.random.default_rng(0)

    def run(n):
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=wl.causal,
                 kv_scale=wl.kv_scale, rows=rows)
        dt = time.perf_counter() - t0
        H, s_q = wl.num_heads, wl.s_q
        flops = 0
        for r in rows:
            b, i = int(r) // (s_q * H), (int(r) // H) % s_q
            L = int(wl.seqlens[b])
            n = (L - s_q + 1 + i) if wl.causal else L
            flops += n * pair_flops_absorb(1)
        return len(rows), dt, flops

    n0, dt0, _ = run(max(8, O.num_threads()))
    n = int(min(total, max(n0, n0 * target_s / max(dt0, 1e-3))))
    n, dt, flops = run(n)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{n} of {total} query rows (fp64, {dt:.1f} s)"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        return 2
    if args.copy_probe:
        return copy_probe()
    import numpy as np
    import torch
    import workloads as W
    import mla_latent_kv_fwd_amd as M

    name = args.config or W.HEADLINE
    wl = W.make_config(name)
    dev = torch.device("cuda")
    kv_np = wl.cache.view(np.int16) if wl.cache.dtype == np.uint16 else wl.cache
    kv_bytes_total = wl.cache.nbytes + (0 if wl.kv_scale is None else wl.kv_scale.nbytes)
    copies = args.copies or max(1, math.ceil(2 * MALL_BYTES / kv_bytes_total))
    kvs = [torch.from_numpy(kv_np).to(dev) for _ in range(copies)]
    kss = [None if wl.kv_scale is None else torch.from_numpy(wl.kv_scale).to(dev) for _ in range(copies)]
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seqlens).to(dev)
    dec = M.MlaDecode(batch=wl.batch, seqlen_q=wl.s_q, num_heads=wl.num_heads, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], causal=wl.causal,
                      kv_dtype=M.MLA_KV_FP8_E4M3FN if wl.kv_dtype == "fp8_e4m3fn" else M.MLA_KV_BF16,
                      softmax_scale=float(wl.softmax_scale))
    stream = torch.cuda.current_stream()

    # Event pairs cost GPU time on this stack (each recorded pair adds several us to
    # the step it sits in), so inside the timed region only the attention kernel --
    # the one the roofline describes -- is bracketed, and only on every
    # --event-every'th step; the plan and combine are timed in a separate pass.
    def step(i, ev=None, all_kernels=False):
        if ev is not None and all_kernels:
            ev[0].record(stream)
        dec.plan(sl)
        if ev is not None:
            ev[1].record(stream)
        dec.decode(q, kvs[i % copies], bt, sl, kss[i % copies])
        if ev is not None:
            ev[2].record(stream)
        dec.combine()
        if ev is not None and all_kernels:
            ev[3].record(stream)

    every = max(1, args.event_every)
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in range(0, args.steps, every)}
    # Warm-up: the W steps asked for, then untimed steps until the GPU has been busy
    # for WARM_SECONDS (clock ramp), ending right before the timed region.
    for i in range(args.warmup):
        step(i)
    warm_total = args.warmup + keep_busy(torch, lambda i: step(i), seconds=args.warm_seconds, min_calls=0)

    # Timed region: exactly `steps` steps, synchronised on both sides.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs.values()]

    # Per-kernel breakdown (outside the timed region): events around every kernel.
    nb = min(args.steps, 50)
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nb)]
    for i in range(nb):
        step(i, evb[i], all_kernels=True)
    torch.cuda.synchronize()
    plan_ms = [e[0].elapsed_time(e[1]) for e in evb]
    comb_ms = [e[2].elapsed_time(e[3]) for e in evb]
    ms_per_step = wall * 1e3 / args.steps
    flops, kv_bytes, alg_bytes = workload_counts(wl.seqlens, wl.num_heads, wl.s_q, wl.causal, wl.kv_dtype)
    dec_avg = float(np.mean(dec_ms))
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kv_gbps = kv_bytes / (ms_per_step * 1e-3) / 1e9
    dec_gbps = alg_bytes / (dec_avg * 1e-3) / 1e9
    dec_tflops = flops / (dec_avg * 1e-3) / 1e12
    mfma_bound = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) > alg_bytes / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(dec_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dec_tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": measured_traffic(name, wl.kv_dtype)}
    else:
        roof = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(name, wl.kv_dtype)}
    flags = dec.flags()
    line = {
        "metric": "MLA decode TFLOP/s + effective KV GB/s (% roofline), B=64 H=128 L=4096 bf16",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_note": f"{warm_total} untimed steps in all: the W asked for, then more until the GPU had been "
                       f"busy {args.warm_seconds} s (clock ramp-up from idle)",
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "batch": wl.batch, "heads": wl.num_heads, "seqlen_q": wl.s_q,
                   "seqlens_sum": int(wl.seqlens.sum()), "kv_dtype": wl.kv_dtype, "page": 64, "cache_copies": copies},
        "kv_gbps": round(kv_gbps, 1), "kv_frac_hbm": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "tflops_frac_mfma": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "kernel_ms": {"plan": round(float(np.mean(plan_ms)), 5), "decode": round(dec_avg, 5),
                      "combine": round(float(np.mean(comb_ms)), 5)},
        "kernel_timing": f"decode: HIP events inside the timed region on every {every}th step "
                         f"({len(dec_ms)} launches); plan, combine: a separate pass after it",
        "roofline": roof,
        "flags": flags,
    }
    if not args.no_proj:
        del kvs, kss
        line["projections"] = bench_projections(torch, M, W, wl.batch * wl.s_q, wl.num_heads)
    if not args.no_prefill:
        line["prefill"] = bench_prefill(torch, M, W, args.prefill)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
