#!/usr/bin/env python3
"""Benchmark of one MLA absorb-path decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--copies C] [--no-cpu] [--no-configs]

A step is one decode of one layer over one batch of synthetic inputs already
resident in HBM: the attention kernel over the paged cache and the LSE combine
of the split requests.  The split plan is computed once per model step from the
sequence lengths and serves every layer, so it runs once before the timed
region and is timed on its own (``kernel_ms.plan``; ``ms_per_step_with_plan``
adds it to the step).  The timed region holds exactly K steps between device
synchronisations.  The cache is cycled over C independent copies so repeats
cannot be served from the 256 MB last-level cache (C is chosen so the copies
total at least twice that, unless given); ``warm_single_copy`` repeats the
step on one copy, labelled as such.

Prints one JSON line.  ``value`` is algorithmic TFLOP/s of the step on the
headline workload (or --config); ``roofline`` describes the attention kernel
alone: its average duration over at least 100 back-to-back launches between
one HIP event pair on the stream it runs on; ``parity`` compares the step's
output with the fp64 oracle on the rows of ``cpu_baseline``'s sample;
``configs`` repeats the measurement on the other measured workloads (ragged
batch, two new tokens, FP8 cache on both of its routes) with parity on sampled
rows; ``projections``
times the two per-head projections on either side of the step and ``prefill``
the chunked expand path on 512 new tokens after a 32K prefix.  Step times are
reported as the mean over the timed region and as p10 / p50 / p90 of blocks of
10 steps.  Every timed leg starts after the GPU has been kept busy for a
while, so that its clocks have left the idle state.
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
FP8_MFMA_PEAK_TFLOPS = 5000.0     # MI355X dense fp8
MALL_BYTES = 256 << 20            # last-level (Infinity) cache
D_LATENT, D_ROPE, D_NOPE, D_V = 512, 64, 128, 128


# ---------------------------------------------------------------- algorithmic accounting
# Counted from the contractions the kernels perform.  For one visible cached token and all H heads of one new
# token, the absorb path forms a D_QK-wide score per head (QK^T) and adds a D_LATENT-wide weighted row per head (PV),
# a multiply-add counting 2 FLOPs.  tests/test_bench_accounting.py checks these counts against the figures the
# handbook prints ("MLA inference: two computation paths and FlashMLA", section "Which is faster: count new tokens
# and cached tokens").
D_QK = D_LATENT + D_ROPE


def visible_keys(L, s_q, causal):
    """Cached tokens each of the s_q new-token rows of a request attends to.  L counts the new tokens themselves;
    with the causal mask, new token i (0-based) sees every earlier token and itself: L - s_q + 1 + i keys."""
    return [L - s_q + 1 + i if causal else L for i in range(s_q)]


def decode_flops_per_key(H):
    """One visible key for the H heads of one new token: a D_QK-wide dot product (score) and a D_LATENT-wide
    weighted row (value) per head."""
    return H * (2 * D_QK + 2 * D_LATENT)


def kv_bytes_per_token(kv_dtype="bf16"):
    """Bytes of one cached token: its D_QK stored numbers (2 bytes each in bf16; 1 byte each in E4M3FN, plus the
    token's fp32 scale)."""
    return D_QK * 2 if kv_dtype == "bf16" else D_QK + 4


def workload_counts(seqlens, H, s_q, causal, kv_dtype="bf16"):
    """(FLOPs, KV bytes, total algorithmic bytes) of one decode step over these requests.  The total adds q~ read
    once, the bf16 output and fp32 LSE written once, and the block-table entries and lengths read."""
    keys = sum(sum(visible_keys(int(L), s_q, causal)) for L in seqlens)
    flops = keys * decode_flops_per_key(H)
    kv = sum(int(L) for L in seqlens) * kv_bytes_per_token(kv_dtype)
    B = len(seqlens)
    io = B * s_q * H * (D_QK * 2 + D_LATENT * 2 + 4)
    tables = B * 4 + sum(-(-int(L) // 64) for L in seqlens) * 4
    return flops, kv, kv + io + tables


def expansion_flops_per_token(H):
    """The expand path's per-head products of one cached latent: W_UK[h] (D_NOPE x D_LATENT) and W_UV[h]
    (D_V x D_LATENT) applied to the D_LATENT-wide latent."""
    return H * 2 * D_LATENT * (D_NOPE + D_V)


def mha_flops_per_key(H):
    """One (query, key) pair of the expand path's attention: a (D_NOPE + D_ROPE)-wide score and a D_V-wide
    weighted row per head."""
    return H * (2 * (D_NOPE + D_ROPE) + 2 * D_V)


def projection_flops_per_token(H):
    """The absorb path's two per-head projections of one new token: q^N (D_NOPE) through W_UK[h]^T to the
    D_LATENT-wide absorbed query, and the D_LATENT-wide latent output through W_UV[h] to D_V."""
    return H * 2 * D_LATENT * (D_NOPE + D_V)


# ---------------------------------------------------------------- benchmark
def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None)
    ap.add_argument("--fp8-path", default="exact", choices=("exact", "mfma"),
                    help="route for an FP8 cache: exact (bf16 MFMAs) or mfma (E4M3 MFMAs)")
    ap.add_argument("--copies", type=int, default=0, help="independent cache copies to cycle (0 = auto)")
    ap.add_argument("--block", type=int, default=10, help="steps per event-timed block (percentiles)")
    ap.add_argument("--roofline-launches", type=int, default=200,
                    help="back-to-back attention launches timed for the roofline (at least 100)")
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="keep the GPU busy this long after the W warm-up steps (0 for counter runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the parity check")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the CPU baseline sample")
    ap.add_argument("--no-configs", action="store_true", help="measure only the main workload")
    ap.add_argument("--config-steps", type=int, default=200, help="timed steps for each of the other workloads")
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


ROUTE_SOURCES = {"exact": ("mla_decode_kernel.hip", "mla_decode_common.h"),
                 "mfma": ("mla_decode_fp8mfma.hip", "mla_decode_common.h")}


def kernel_source_digest(route="exact"):
    """sha256 over the attention kernel's device sources of one route (the file that holds it, then the shared
    device helpers)."""
    import hashlib
    h = hashlib.sha256()
    for name in ROUTE_SOURCES[route]:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_kv_fwd_amd", "csrc", name),
                  "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, route="exact"):
    """HBM bytes per attention-kernel launch from the committed counter summary of this workload (and route), or
    None when there is none or the kernel's sources changed since the counters were taken."""
    suffix = "" if route == "exact" else "_fp8mfma"
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}{suffix}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip().strip("`")] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_digest(route):
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
    """Algorithmic FLOPs of the expand path for n new tokens after L - n cached ones: the expansion of each of the
    L cached latents into per-head keys and values, plus the attention over every visible (query, key) pair."""
    return L * expansion_flops_per_token(H) + sum(visible_keys(L, n, True)) * mha_flops_per_key(H)


def bench_prefill(torch, M, W, name, launches=10):
    """The chunked expand path (mla_chunked_prefill) on one of the handbook's shapes: average time per call
    over back-to-back calls between one event pair, after the timed region."""
    import numpy as np
    cfg = PREFILL_WORKLOADS[name]
    H, n, L = cfg["num_heads"], cfg["num_new"], cfg["seqlen"]
    pw = W.make_prefill_workload(name, num_heads=H, num_new=n, seqlen=L, seed=1, poison=False)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
    q, kv, bt, wuk, wuv = dev(pw.q), dev(pw.cache), dev(pw.block_table), dev(pw.w_uk), dev(pw.w_uv)
    flops = prefill_counts(H, n, L)

    def timed(chunk_tokens):
        pre = M.MlaPrefill(num_heads=H, num_new=n, seqlen=L, num_pages=pw.num_pages, max_blocks=len(pw.block_table),
                           chunk_tokens=chunk_tokens)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        keep_busy(torch, lambda i: pre(q, kv, bt, wuk, wuv), seconds=0.1, min_calls=3)
        e0.record()
        for _ in range(launches):
            pre(q, kv, bt, wuk, wuv)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        tflops = flops / (ms * 1e-3) / 1e12
        del pre
        return {"chunk_tokens": chunk_tokens, "ms": round(ms, 4), "tflops": round(tflops, 1),
                "frac_mfma": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}

    res = {"workload": name, "heads": H, "new_tokens": n, "seqlen": L, "gflop": round(flops / 1e9, 1)}
    res.update(timed(cfg["chunk_tokens"]))
    whole = -(-L // 64) * 64
    if whole != cfg["chunk_tokens"]:
        # The same call with the whole context expanded at once (its K and V take
        # L x H x 640 bytes: 2.7 GB for the extend, which HBM holds easily).
        res["one_chunk"] = timed(whole)
    res["timing"] = (f"{launches} back-to-back calls between one event pair per chunk size, after the timed region; "
                     "not part of the step")
    return res


def oracle_rows(wl, rows):
    """fp64 oracle output and LSE of the given flat (request, new token, head) rows, and the seconds it took."""
    from oracle import oracle as O
    t0 = time.perf_counter()
    o, l = O.attend(wl.q, wl.cache, wl.block_table, wl.seqlens, softmax_scale=wl.softmax_scale, causal=wl.causal,
                    kv_scale=wl.kv_scale, rows=rows)
    return o, l, time.perf_counter() - t0


def rows_flops(wl, rows):
    H, s_q = wl.num_heads, wl.s_q
    return sum(visible_keys(int(wl.seqlens[int(r) // (s_q * H)]), s_q, wl.causal)[(int(r) // H) % s_q] *
               decode_flops_per_key(1) for r in rows)


def cpu_baseline(wl, target_s):
    """fp64 oracle on a bounded sample of rows, sized to take about target_s seconds on the host's cores.
    Returns the dict for the JSON line and (rows, out, lse) for the parity check."""
    import numpy as np
    from oracle import oracle as O
    total = wl.batch * wl.s_q * wl.num_heads
    rng = np.random.default_rng(0)
    pick = lambda n: np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)
    rows = pick(max(8, O.num_threads()))
    _, _, dt0 = oracle_rows(wl, rows)
    n = int(min(total, max(len(rows), len(rows) * target_s / max(dt0, 1e-3))))
    rows = pick(n)
    o, l, dt = oracle_rows(wl, rows)
    res = {"value": round(rows_flops(wl, rows) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": O.num_threads(),
           "kind": "oracle", "sample": f"{len(rows)} of {total} query rows of {wl.name} (fp64, {dt:.1f} s)"}
    return res, (rows, o, l)


def parity(M, W, out, lse, rows, ref_o, ref_l, bf16_tol=True):
    """Output and LSE of the GPU step on these rows against the oracle's (the tests' tolerances)."""
    import numpy as np
    got = W.bf16_bits_to_f32(out.reshape(-1, M.HEAD_DIM_V)[rows]).astype(np.float64)
    gl = lse.reshape(-1)[rows].astype(np.float64)
    d = got - ref_o
    per_row = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(ref_o, axis=1), 1e-30)
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref_o), 1e-30))
    mx = float(np.abs(d).max())
    lerr = float(np.abs(gl - ref_l).max())
    ok = rel <= 5e-3 and mx <= 2e-2 and lerr <= 1e-3 if bf16_tol else rel <= 3e-2
    return {"rows": int(len(rows)), "of": int(out.reshape(-1, M.HEAD_DIM_V).shape[0]), "out_max_abs": mx,
            "out_rel_l2": rel, "worst_row_rel_l2": float(per_row.max()), "worst_row": int(rows[int(per_row.argmax())]),
            "lse_max_abs": lerr, "within_tolerance": bool(ok)}


GRAPH_STEPS = 10


def graph_step_ms(torch, step, copies, steps):
    """Average time per step when GRAPH_STEPS steps, cycling the cache copies, are captured into one HIP graph
    and the graph is replayed until about `steps` steps have run (after two warm-up replays).  The library only
    launches kernels (no allocation, memset or synchronisation), so the step can be captured."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(GRAPH_STEPS):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(GRAPH_STEPS):
            step(i)
    reps = max(1, steps // GRAPH_STEPS)
    for _ in range(2):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * GRAPH_STEPS)
    del g
    return ms


def input_digest(wl):
    """sha256 over the workload's inputs as the kernels read them (q~, the cache, its scales, the block table and
    the lengths), so two runs can be checked to have measured the same data."""
    import hashlib
    import numpy as np
    h = hashlib.sha256()
    for x in (wl.q, wl.cache, wl.kv_scale, wl.block_table, wl.seqlens):
        if x is not None:
            h.update(memoryview(np.ascontiguousarray(x)).cast("B"))
    return h.hexdigest()[:16]


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 5), "p50": round(float(np.percentile(a, 50)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def roofline_of(flops, alg_bytes, kernel_ms, traffic, mfma_peak=BF16_MFMA_PEAK_TFLOPS):
    """Binding roofline of the attention kernel: whichever of HBM bytes and MFMA time (at the peak of the
    kernel's MFMA type) is larger."""
    gbps = alg_bytes / (kernel_ms * 1e-3) / 1e9
    tfl = flops / (kernel_ms * 1e-3) / 1e12
    if flops / (mfma_peak * 1e12) > alg_bytes / (HBM_PEAK_GBPS * 1e9):
        return {"bound": "mfma", "achieved": round(tfl, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tfl / mfma_peak, 4), "traffic": traffic}
    return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}


def measure(torch, M, W, name, *, steps, warmup, warm_seconds, copies=0, block=10, roof_launches=200,
            parity_rows=None, plan_launches=50, fp8_path="exact"):
    """Time one workload: plan once; W warm-up steps and warm_seconds of untimed ones; exactly `steps` timed steps
    (decode + combine) between synchronisations; then the attention kernel alone for the roofline, the plan alone,
    the combine alone, and the step on a single cache copy.  Returns (dict, workload, out, lse)."""
    import numpy as np
    wl = W.make_config(name)
    dev = torch.device("cuda")
    kv_np = wl.cache.view(np.int16) if wl.cache.dtype == np.uint16 else wl.cache
    kv_bytes_total = wl.cache.nbytes + (0 if wl.kv_scale is None else wl.kv_scale.nbytes)
    copies = copies or max(1, math.ceil(2 * MALL_BYTES / kv_bytes_total))
    kvs = [torch.from_numpy(kv_np).to(dev) for _ in range(copies)]
    kss = [None if wl.kv_scale is None else torch.from_numpy(wl.kv_scale).to(dev) for _ in range(copies)]
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seqlens).to(dev)
    fp8 = wl.kv_dtype == "fp8_e4m3fn"
    route = fp8_path if fp8 else "exact"
    dec = M.MlaDecode(batch=wl.batch, seqlen_q=wl.s_q, num_heads=wl.num_heads, num_pages=wl.num_pages,
                      max_blocks_per_seq=wl.block_table.shape[1], causal=wl.causal,
                      kv_dtype=M.MLA_KV_FP8_E4M3FN if fp8 else M.MLA_KV_BF16, softmax_scale=float(wl.softmax_scale),
                      fp8_path=M.MLA_FP8_PATH_MFMA if route == "mfma" else M.MLA_FP8_PATH_EXACT)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    dec.plan(sl)   # once: the plan depends only on the lengths and serves every step

    def step(i, c=None):
        k = i % copies if c is None else c
        dec.decode(q, kvs[k], bt, sl, kss[k])
        dec.combine()

    for i in range(warmup):
        step(i)
    warm_total = warmup + keep_busy(torch, step, seconds=warm_seconds, min_calls=0)

    # Timed region: exactly `steps` steps, synchronised on both sides; an event at every block boundary.
    block = max(1, min(block, steps))
    nblk = max(1, steps // block)
    marks = [ev() for _ in range(nblk + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % block == 0 and i // block <= nblk:
            marks[i // block].record(stream)
        step(i)
    if steps % block == 0:
        marks[nblk].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    blocks = [marks[j].elapsed_time(marks[j + 1]) / block for j in range(nblk) if (j + 1) * block <= steps]
    ms_per_step = wall * 1e3 / steps
    out_np = dec.out.view(torch.int16).cpu().numpy().view(np.uint16)
    lse_np = dec.lse.cpu().numpy()
    flags = dec.flags()

    # The attention kernel alone: back-to-back launches between one event pair (roofline).
    R = max(100, roof_launches)
    keep_busy(torch, step, seconds=0.05, min_calls=0)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for i in range(R):
        dec.decode(q, kvs[i % copies], bt, sl, kss[i % copies])
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / R
    # The plan alone and the combine alone (back-to-back launches; the combine re-merges the same pieces).
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(plan_launches):
        dec.plan(sl)
    e1.record(stream)
    torch.cuda.synchronize()
    plan_ms = e0.elapsed_time(e1) / plan_launches
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(plan_launches):
        dec.combine()
    e1.record(stream)
    torch.cuda.synchronize()
    comb_ms = e0.elapsed_time(e1) / plan_launches
    # The step on one cache copy (partly served by the last-level cache: labelled, not the headline).
    keep_busy(torch, lambda i: step(i, 0), seconds=0.05, min_calls=0)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for i in range(steps):
        step(i, 0)
    e1.record(stream)
    torch.cuda.synchronize()
    warm1_ms = e0.elapsed_time(e1) / steps
    graph_ms = graph_step_ms(torch, step, copies, steps)

    flops, kv_bytes, alg_bytes = workload_counts(wl.seqlens, wl.num_heads, wl.s_q, wl.causal, wl.kv_dtype)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kv_gbps = kv_bytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "workload": name, "batch": wl.batch, "heads": wl.num_heads, "seqlen_q": wl.s_q, "causal": wl.causal,
        "seqlens_sum": int(wl.seqlens.sum()), "kv_dtype": wl.kv_dtype, "page": 64, "cache_copies": copies,
        "input_sha256": input_digest(wl),
        "route": route if fp8 else "bf16",
        "steps": steps, "warmup_steps_total": warm_total, "ms_per_step": round(ms_per_step, 5),
        "step_ms": percentiles(blocks), "ms_per_step_with_plan": round(ms_per_step + plan_ms, 5),
        "tflops": round(tflops, 2), "tflops_frac_mfma": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "kv_gbps": round(kv_gbps, 1), "kv_frac_hbm": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "gflop": round(flops / 1e9, 3), "kv_mb": round(kv_bytes / 1e6, 2), "alg_mb": round(alg_bytes / 1e6, 2),
        "kernel_ms": {"decode": round(dec_ms, 5), "combine": round(comb_ms, 5), "plan": round(plan_ms, 5)},
        "roofline": roofline_of(flops, alg_bytes, dec_ms, measured_traffic(name, route),
                                FP8_MFMA_PEAK_TFLOPS if route == "mfma" else BF16_MFMA_PEAK_TFLOPS),
        "warm_single_copy": {"ms_per_step": round(warm1_ms, 5),
                             "tflops": round(flops / (warm1_ms * 1e-3) / 1e12, 2),
                             "note": "one cache copy reused every step: partly served by the last-level cache"},
        "graph_replay": {"ms_per_step": round(graph_ms, 5), "tflops": round(flops / (graph_ms * 1e-3) / 1e12, 2),
                         "note": f"the same kernels launched from one HIP graph holding {GRAPH_STEPS} captured "
                                 "steps (cycling the cache copies); reported beside the eager stream launches "
                                 "that ms_per_step times"},
        "flags": flags,
    }
    if parity_rows:
        rng = np.random.default_rng(123)
        total = wl.batch * wl.s_q * wl.num_heads
        rows = np.unique(np.concatenate([rng.integers(0, total, parity_rows), [0, total - 1]])).astype(np.int64)
        ro, rl, _ = oracle_rows(wl, rows)
        res["parity"] = parity(M, W, out_np, lse_np, rows, ro, rl, bf16_tol=not fp8)
        res["parity"]["tolerance"] = "rel-L2 <= 3e-2" if fp8 else "rel-L2 <= 5e-3, max-abs <= 2e-2, lse <= 1e-3"
    del kvs, kss
    return res, wl, out_np, lse_np


# (workload, FP8 route): the FP8 workload is measured on both routes, the E4M3-MFMA one under its own key.
OTHER_CONFIGS = (("ragged_b128_h128_l128_32768", "exact"), ("mtp_b32_h128_sq2_l8192", "exact"),
                 ("fp8_b128_h128_l16384", "exact"), ("fp8_b128_h128_l16384", "mfma"))


def main():
    args = _parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU (a single MI355X); --gpus must be 1"}))
        return 2
    if args.copy_probe:
        return copy_probe()
    import torch
    import workloads as W
    import mla_latent_kv_fwd_amd as M

    name = args.config or W.HEADLINE
    main_res, wl, out_np, lse_np = measure(torch, M, W, name, steps=args.steps, warmup=args.warmup,
                                           warm_seconds=args.warm_seconds, copies=args.copies, block=args.block,
                                           roof_launches=args.roofline_launches, fp8_path=args.fp8_path)
    r = main_res
    line = {
        "metric": "MLA decode TFLOP/s + effective KV GB/s (% roofline), B=64 H=128 L=4096 bf16",
        "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_note": f"{r['warmup_steps_total']} untimed steps in all: the W asked for, then more until the GPU "
                       f"had been busy {args.warm_seconds} s (clock ramp-up from idle)",
        "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if r.get("route") == "mfma" else "bf16", "data": "synthetic",
        "config": {k: r[k] for k in ("workload", "batch", "heads", "seqlen_q", "seqlens_sum", "kv_dtype", "page",
                                     "cache_copies", "input_sha256")},
        "step": "decode + combine of one layer; the plan runs once per model step (kernel_ms.plan)",
        "step_ms": r["step_ms"], "ms_per_step_with_plan": r["ms_per_step_with_plan"],
        "kv_gbps": r["kv_gbps"], "kv_frac_hbm": r["kv_frac_hbm"], "tflops_frac_mfma": r["tflops_frac_mfma"],
        "kernel_ms": r["kernel_ms"],
        "kernel_timing": f"decode: {max(100, args.roofline_launches)} back-to-back launches between one HIP event "
                         "pair on its stream; plan, combine: 50 back-to-back launches each",
        "roofline": r["roofline"], "warm_single_copy": r["warm_single_copy"], "graph_replay": r["graph_replay"],
        "flags": r["flags"],
    }
    if not args.no_cpu:
        cb, (rows, ro, rl) = cpu_baseline(wl, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["parity"] = parity(M, W, out_np, lse_np, rows, ro, rl, bf16_tol=wl.kv_dtype == "bf16")
    del wl, out_np, lse_np
    if not args.no_configs and args.config is None:
        line["configs"] = {}
        for cname, route in OTHER_CONFIGS:
            cres, *_ = measure(torch, M, W, cname, steps=args.config_steps, warmup=5, warm_seconds=0.1,
                               block=args.block, roof_launches=100, parity_rows=None if args.no_cpu else 64,
                               fp8_path=route)
            line["configs"][cname if route == "exact" else f"{cname}+fp8_mfma_route"] = cres
    if not args.no_proj:
        line["projections"] = bench_projections(torch, M, W, r["batch"] * r["seqlen_q"], r["heads"])
    if not args.no_prefill:
        line["prefill"] = bench_prefill(torch, M, W, args.prefill)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
