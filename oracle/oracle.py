"""fp64 CPU oracle for MLA absorb-path decode -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and its
binding) never does, and this module imports nothing from it.

Two independent implementations live here:

* ``attend`` / ``lse_merge`` wrap ``mla_oracle.c``: the absorb path, plain
  loops in double precision (see that file's header for the passages each step
  follows).
* ``expand_attention`` is the *expand* path in NumPy float64: per-head keys and
  values are rebuilt from the latent with W_UK and W_UV (``expand_kv``) and an
  ordinary multi-head attention with 192-wide queries/keys and 128-wide values
  is run (``mha_attend``) ("MLA inference: two computation paths and
  FlashMLA", section "Two equivalent paths", path one).  The handbook shows
  both paths give the same output; tests use that equivalence to pin the
  absorb oracle, and with it these two functions.
* ``absorb_q`` / ``project_out`` are the two projections of the absorb path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
# ORACLE_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer (gcc's runtimes must then
# be preloaded into the process; tests/test_sanitizers.py does that in a child process).
_SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_asan.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

Q_BF16, Q_F64 = 0, 1
KV_BF16, KV_E4M3FN = 0, 1
_STATUS = {0: "ok", -1: "bad argument", -2: "block table entry outside the cache",
           -3: "seqlen outside [s_q, max_blocks * page_size]", -4: "out of memory"}


class _Shape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "seqlen_q", "num_heads", "d_latent", "d_rope", "page_size", "num_pages",
        "max_blocks", "causal", "q_dtype", "kv_dtype")] + [("softmax_scale", ctypes.c_float)]


def build(force: bool = False) -> str:
    """Compile mla_oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                               *(_SAN_FLAGS if _SANITIZE else []), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_mla_attend.restype = ctypes.c_int
        lib.oracle_mla_attend.argtypes = [ctypes.POINTER(_Shape)] + [ctypes.c_void_p] * 8 + [ctypes.c_int64] + \
            [ctypes.c_void_p] * 2
        lib.oracle_lse_merge.restype = ctypes.c_int
        lib.oracle_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 4
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_num_threads())


def bf16_to_f64(bits: int) -> float:
    return float(_load().oracle_bf16_to_f64(int(bits)))


def e4m3fn_to_f64(code: int) -> float:
    return float(_load().oracle_e4m3fn_to_f64(int(code)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attend(q, cache, block_table, seqlens, *, softmax_scale, causal=False, kv_scale=None,
           d_rope=64, t_begin=None, t_end=None, rows=None):
    """Absorb-path attention in fp64 over a paged latent cache.

    q:           uint16 bf16 bits or float64, [B, s_q, H, d_latent + d_rope]
    cache:       uint16 bf16 bits or uint8 E4M3FN codes, [P, page, d_latent + d_rope]
    kv_scale:    float32 [P, page] for an E4M3FN cache, else None
    block_table: int32 [B, max_blocks]; seqlens: int32 [B] (counting the new tokens)
    t_begin/t_end: optional int32 [B] token window (split mode); rows: optional flat row ids

    Returns (out float64 [nrows, d_latent], lse float64 [nrows]); without ``rows``
    they are reshaped to [B, s_q, H, d_latent] and [B, s_q, H].
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    cache = np.ascontiguousarray(cache)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    B, s_q, H, D = q.shape
    P, page, Dc = cache.shape
    if Dc != D:
        raise ValueError(f"query width {D} != cache row width {Dc}")
    if q.dtype == np.float64:
        q_dtype = Q_F64
    elif q.dtype == np.uint16:
        q_dtype = Q_BF16
    else:
        raise TypeError("q must be uint16 (bf16 bits) or float64")
    if cache.dtype == np.uint16:
        kv_dtype = KV_BF16
    elif cache.dtype == np.uint8:
        kv_dtype = KV_E4M3FN
        if kv_scale is None:
            raise ValueError("an E4M3FN cache needs kv_scale")
        kv_scale = np.ascontiguousarray(kv_scale, dtype=np.float32)
        if kv_scale.shape != (P, page):
            raise ValueError("kv_scale must be [P, page]")
    else:
        raise TypeError("cache must be uint16 (bf16 bits) or uint8 (E4M3FN codes)")
    shape = _Shape(B, s_q, H, D - d_rope, d_rope, page, P, block_table.shape[1], int(bool(causal)), q_dtype,
                   kv_dtype, float(np.float32(softmax_scale)))
    tb = None if t_begin is None else np.ascontiguousarray(t_begin, dtype=np.int32)
    te = None if t_end is None else np.ascontiguousarray(t_end, dtype=np.int32)
    if rows is None:
        nrows = B * s_q * H
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.shape[0]
    out = np.empty((nrows, D - d_rope), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    st = lib.oracle_mla_attend(ctypes.byref(shape), _ptr(q), _ptr(cache), _ptr(kv_scale), _ptr(block_table),
                               _ptr(seqlens), _ptr(tb), _ptr(te), _ptr(rows_arr), nrows, _ptr(out), _ptr(lse))
    if st != 0:
        raise ValueError(f"oracle_mla_attend: {_STATUS.get(st, st)}")
    if rows is None:
        return out.reshape(B, s_q, H, D - d_rope), lse.reshape(B, s_q, H)
    return out, lse


def lse_merge(out_parts, lse_parts):
    """Merge partial (out_j, lse_j) over disjoint windows: out_parts [J, rows, dv], lse_parts [J, rows]."""
    out_parts = np.ascontiguousarray(out_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    J, R, dv = out_parts.shape
    out = np.empty((R, dv), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    st = _load().oracle_lse_merge(J, R, dv, _ptr(out_parts), _ptr(lse_parts), _ptr(out), _ptr(lse))
    if st != 0:
        raise ValueError(f"oracle_lse_merge: {_STATUS.get(st, st)}")
    return out, lse


def absorb_q(q_nope, q_rope, w_uk):
    """Absorbed query in float64: q~[t,h] = [W_UK[h]^T q^N[t,h] ; q^R[t,h]].

    q_nope [T, H, dn], q_rope [T, H, dr], w_uk [H, dn, d_latent] (k^N = W_UK[h] c).
    ("MLA inference: two computation paths and FlashMLA", section "Two
    equivalent paths", path two: W_UK folded into the query.)  Returns
    [T, H, d_latent + dr], latent part first.
    """
    q_lat = np.einsum("thn,hnc->thc", np.asarray(q_nope, np.float64), np.asarray(w_uk, np.float64))
    return np.concatenate([q_lat, np.asarray(q_rope, np.float64)], axis=-1)


def project_out(o_latent, w_uv):
    """Output projection in float64: out[t,h] = W_UV[h] o[t,h].

    o_latent [T, H, d_latent] (the latent-space attention output), w_uv
    [H, dv, d_latent] (v = W_UV[h] c).  (Same passage: W_UV applied after the
    attention.)  Returns [T, H, dv].
    """
    return np.einsum("thc,hvc->thv", np.asarray(o_latent, np.float64), np.asarray(w_uv, np.float64))


def expand_kv(latent, k_rope, w_uk, w_uv):
    """Expand path, first step, in float64: per-head keys and values rebuilt from the cache.

    latent [T, d_latent], k_rope [T, dr], w_uk and w_uv [H, dn|dv, d_latent] (k^N = W_UK[h] c).
    Returns k [H, T, dn + dr] (k^N[h,t] then the shared k^R[t]) and v [H, T, dv].
    ("MLA inference: two computation paths and FlashMLA", section "Two equivalent paths", path one.)
    """
    latent = np.asarray(latent, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    k_nope = np.stack([latent @ w_uk[h].T for h in range(w_uk.shape[0])])   # [H, T, dn]
    v = np.stack([latent @ w_uv[h].T for h in range(w_uv.shape[0])])        # [H, T, dv]
    H, T = k_nope.shape[0], k_nope.shape[1]
    k = np.concatenate([k_nope, np.broadcast_to(k_rope[None], (H, T, k_rope.shape[1]))], axis=-1)
    return k, v


def mha_attend(q, k, v, softmax_scale, query_pos, key_pos):
    """Ordinary multi-head attention in float64 with a causal rule on absolute positions.

    q [Tq, H, dqk], k [H, Tk, dqk], v [H, Tk, dv]; query at position p sees keys at positions <= p.
    Returns (out [Tq, H, dv], lse [Tq, H]); a query that sees no key gets out 0 and lse -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    logits = np.einsum("qhd,htd->hqt", q, np.asarray(k, np.float64)) * softmax_scale
    visible = np.asarray(key_pos)[None, :] <= np.asarray(query_pos)[:, None]   # [Tq, Tk]
    logits = np.where(visible[None], logits, -np.inf)
    mx = logits.max(axis=-1, keepdims=True)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(logits - safe)
    z = w.sum(axis=-1, keepdims=True)
    out = np.einsum("hqt,htv->qhv", np.divide(w, z, out=np.zeros_like(w), where=z > 0), np.asarray(v, np.float64))
    lse = np.where(z > 0, safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)[..., 0].T   # [Tq, H]
    return out, lse


def expand_attention(q_nope, q_rope, w_uk, w_uv, latent, k_rope, softmax_scale, query_pos, key_pos):
    """Expand path (path one) in float64, for one request: expand_kv, then mha_attend with q = [q^N ; q^R].

    q_nope [Tq, H, dn], q_rope [Tq, H, dr]; w_uk, w_uv [H, dn|dv, d_latent] (k^N = W_UK[h] c);
    latent [Tk, d_latent], k_rope [Tk, dr]; query_pos [Tq] and key_pos [Tk] are absolute
    positions: query at position p sees keys at positions <= p.
    Returns (out [Tq, H, dv], lse [Tq, H]).
    """
    k, v = expand_kv(latent, k_rope, w_uk, w_uv)
    q = np.concatenate([np.asarray(q_nope, np.float64), np.asarray(q_rope, np.float64)], axis=-1)
    return mha_attend(q, k, v, softmax_scale, query_pos, key_pos)
