"""Python binding of libmla_decode.so: MLA absorb-path decode on MI355X (gfx950).

Argument marshalling only.  Every step of the decode runs in the HIP kernels of
the shared library; this module never computes attention itself, and it raises
if the library is missing.  PyTorch supplies device memory and streams.

The entry points carry the names of the C ABI (include/mla_decode.h,
include/mla_proj.h): ``mla_get_workspace``, ``mla_decode_fwd``,
``mla_splitkv_combine``, ``mla_workspace_flags``, ``mla_absorb_q``,
``mla_project_out``.  ``MlaDecode`` wraps the decode step for torch tensors;
``absorb_q`` and ``project_out`` the two projections.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_DECODE_LIB selects another build of the same library (the host-sanitizer build that
# tests/test_sanitizers.py makes); by default the in-tree library.
LIB_PATH = os.environ.get("MLA_DECODE_LIB") or os.path.join(_PKG, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE_TOO_SMALL = -3
MLA_ERR_HIP = -4
MLA_ERR_SCRATCH_TOO_SMALL = -5
MLA_NOALLOC_SCRATCH_BYTES = 80 << 20
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3FN = 1
MLA_FLAG_SEQLEN_CLAMPED = 0x1
MLA_FLAG_BAD_BLOCK = 0x2
MLA_FLAG_BAD_PLAN = 0x4
MLA_FP8_PATH_EXACT = 0
MLA_FP8_PATH_MFMA = 1

HEAD_DIM_QK = 576
HEAD_DIM_V = 512
PAGE_SIZE = 64
SOFTMAX_SCALE = 1.0 / math.sqrt(128 + 64)

EXPORTED_SYMBOLS = ("mla_get_workspace", "mla_decode_fwd", "mla_splitkv_combine", "mla_workspace_flags",
                    "mla_status_string", "mla_absorb_q", "mla_project_out", "mla_expand_kv",
                    "mla_prefill_attention", "mla_lse_merge", "mla_prefill_workspace_size", "mla_chunked_prefill",
                    "mla_decode_noalloc")
D_NOPE, D_ROPE, D_LATENT, D_V = 128, 64, 512, 128


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} ({status})")
        self.status = status


class MlaDeviceError(RuntimeError):
    """Debug mode only: the device-side values of a decode call were invalid (found before the launch by the
    synchronous checks, or reported by the kernels in the workspace flags after it)."""

    def __init__(self, message: str, flags: int = 0):
        super().__init__(message)
        self.flags = flags


_FLAG_TEXT = ((0x1, "a sequence length outside [seqlen_q, max_blocks_per_seq * 64] was clamped"),
              (0x2, "a referenced block-table entry was outside [0, num_pages)"),
              (0x4, "the workspace held no plan for these parameters"))


def describe_flags(flags: int) -> str:
    """The workspace flag bits as text."""
    parts = [t for bit, t in _FLAG_TEXT if flags & bit]
    return "; ".join(parts) if parts else "none"


def debug_from_env() -> bool:
    """MLA_DEBUG=1 in the environment turns on MlaDecode's debug mode by default."""
    return os.environ.get("MLA_DEBUG", "") not in ("", "0")


class DecodeParams(ctypes.Structure):
    """Mirror of mla_decode_params."""
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("num_workgroups", ctypes.c_int32),
                ("fp8_path", ctypes.c_int32)]


class ProjParams(ctypes.Structure):
    """Mirror of mla_proj_params."""
    _fields_ = [("tokens", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_latent", ctypes.c_int32), ("d_v", ctypes.c_int32)]


def make_proj_params(*, tokens, num_heads, d_nope=D_NOPE, d_rope=D_ROPE, d_latent=D_LATENT, d_v=D_V) -> ProjParams:
    return ProjParams(tokens, num_heads, d_nope, d_rope, d_latent, d_v)


class PrefillParams(ctypes.Structure):
    """Mirror of mla_prefill_params."""
    _fields_ = [("num_heads", ctypes.c_int32), ("num_new", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_v", ctypes.c_int32)]


def make_prefill_params(*, num_heads, num_new, seqlen, num_pages, max_blocks, chunk_tokens=4096,
                        softmax_scale=1.0 / math.sqrt(D_NOPE + D_ROPE), d_nope=D_NOPE, d_rope=D_ROPE,
                        d_latent=D_LATENT, d_v=D_V) -> PrefillParams:
    return PrefillParams(num_heads, num_new, seqlen, num_pages, max_blocks, chunk_tokens, softmax_scale, d_nope,
                         d_rope, d_latent, d_v)


def make_params(*, batch, seqlen_q, num_heads, num_pages, max_blocks_per_seq, kv_dtype=MLA_KV_BF16, causal=False,
                softmax_scale=SOFTMAX_SCALE, num_workgroups=0, fp8_path=MLA_FP8_PATH_EXACT, head_dim_qk=HEAD_DIM_QK,
                head_dim_v=HEAD_DIM_V, page_size=PAGE_SIZE) -> DecodeParams:
    return DecodeParams(batch, seqlen_q, num_heads, head_dim_qk, head_dim_v, page_size, num_pages,
                        max_blocks_per_seq, kv_dtype, int(bool(causal)), softmax_scale, num_workgroups, fp8_path)


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mla_latent_kv_fwd_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(DecodeParams)
    lib.mla_get_workspace.argtypes = [pp, vp, vp, ctypes.POINTER(sz), vp]
    lib.mla_decode_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mla_splitkv_combine.argtypes = [pp, vp, sz, vp, vp, vp]
    lib.mla_decode_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mla_workspace_flags.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    ppp = ctypes.POINTER(ProjParams)
    lib.mla_absorb_q.argtypes = [ppp, vp, vp, vp, vp, vp]
    lib.mla_project_out.argtypes = [ppp, vp, vp, vp, vp]
    pfp = ctypes.POINTER(PrefillParams)
    i32 = ctypes.c_int32
    lib.mla_expand_kv.argtypes = [pfp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.mla_prefill_attention.argtypes = [pfp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.mla_lse_merge.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    lib.mla_prefill_workspace_size.argtypes = [pfp, ctypes.POINTER(sz)]
    lib.mla_chunked_prefill.argtypes = [pfp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    for name in EXPORTED_SYMBOLS:
        if name == "mla_status_string":
            continue
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MlaError(fn, status, load_library().mla_status_string(status).decode())


def mla_get_workspace(params: DecodeParams, seqlens_ptr: int = 0, workspace_ptr: int = 0,
                      workspace_bytes: int = 0, stream: int = 0) -> int:
    """Size query (workspace_ptr == 0) or plan launch; returns the required size in bytes."""
    nbytes = ctypes.c_size_t(workspace_bytes)
    _check("mla_get_workspace", load_library().mla_get_workspace(
        ctypes.byref(params), seqlens_ptr or None, workspace_ptr or None, ctypes.byref(nbytes), stream or None))
    return nbytes.value


def mla_decode_fwd(params: DecodeParams, q_ptr: int, kv_ptr: int, kv_scale_ptr: int, block_table_ptr: int,
                   seqlens_ptr: int, workspace_ptr: int, workspace_bytes: int, out_ptr: int, lse_ptr: int,
                   stream: int = 0) -> None:
    _check("mla_decode_fwd", load_library().mla_decode_fwd(
        ctypes.byref(params), q_ptr or None, kv_ptr or None, kv_scale_ptr or None, block_table_ptr or None,
        seqlens_ptr or None, workspace_ptr or None, workspace_bytes, out_ptr or None, lse_ptr or None,
        stream or None))


def mla_splitkv_combine(params: DecodeParams, workspace_ptr: int, workspace_bytes: int, out_ptr: int,
                        lse_ptr: int, stream: int = 0) -> None:
    _check("mla_splitkv_combine", load_library().mla_splitkv_combine(
        ctypes.byref(params), workspace_ptr or None, workspace_bytes, out_ptr or None, lse_ptr or None,
        stream or None))


def mla_decode_noalloc(params: DecodeParams, q_ptr: int, kv_ptr: int, kv_scale_ptr: int, block_table_ptr: int,
                       seqlens_ptr: int, out_ptr: int, lse_ptr: int, stream: int = 0) -> None:
    _check("mla_decode_noalloc", load_library().mla_decode_noalloc(
        ctypes.byref(params), q_ptr or None, kv_ptr or None, kv_scale_ptr or None, block_table_ptr or None,
        seqlens_ptr or None, out_ptr or None, lse_ptr or None, stream or None))


def mla_workspace_flags(workspace_ptr: int, stream: int = 0) -> int:
    flags = ctypes.c_uint32(0)
    _check("mla_workspace_flags", load_library().mla_workspace_flags(workspace_ptr or None, ctypes.byref(flags),
                                                                     stream or None))
    return flags.value


def mla_absorb_q(params: ProjParams, q_nope_ptr: int, q_rope_ptr: int, w_uk_ptr: int, q_tilde_ptr: int,
                 stream: int = 0) -> None:
    _check("mla_absorb_q", load_library().mla_absorb_q(
        ctypes.byref(params), q_nope_ptr or None, q_rope_ptr or None, w_uk_ptr or None, q_tilde_ptr or None,
        stream or None))


def mla_project_out(params: ProjParams, o_latent_ptr: int, w_uv_ptr: int, out_ptr: int, stream: int = 0) -> None:
    _check("mla_project_out", load_library().mla_project_out(
        ctypes.byref(params), o_latent_ptr or None, w_uv_ptr or None, out_ptr or None, stream or None))


def _bf16_tensor(x, shape, name):
    if tuple(x.shape) != tuple(shape) or x.element_size() != 2 or not x.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous 16-bit tensor of shape {tuple(shape)}, got {tuple(x.shape)}")


def absorb_q(q_nope, q_rope, w_uk, out=None):
    """q~ [T, H, 576] bf16 from q^N [T, H, 128], q^R [T, H, 64] and W_UK [H, 128, 512] (all bf16 on the device)."""
    import torch
    T, H = q_nope.shape[0], q_nope.shape[1]
    _bf16_tensor(q_nope, (T, H, D_NOPE), "q_nope")
    _bf16_tensor(q_rope, (T, H, D_ROPE), "q_rope")
    _bf16_tensor(w_uk, (H, D_NOPE, D_LATENT), "w_uk")
    if out is None:
        out = torch.empty((T, H, D_LATENT + D_ROPE), dtype=q_nope.dtype, device=q_nope.device)
    _bf16_tensor(out, (T, H, D_LATENT + D_ROPE), "out")
    mla_absorb_q(make_proj_params(tokens=T, num_heads=H), q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(),
                 out.data_ptr(), torch.cuda.current_stream(q_nope.device).cuda_stream)
    return out


def project_out(o_latent, w_uv, out=None):
    """W_UV[h] o[t,h]: [T, H, 128] bf16 from o [T, H, 512] and W_UV [H, 128, 512] (all bf16 on the device)."""
    import torch
    T, H = o_latent.shape[0], o_latent.shape[1]
    _bf16_tensor(o_latent, (T, H, D_LATENT), "o_latent")
    _bf16_tensor(w_uv, (H, D_V, D_LATENT), "w_uv")
    if out is None:
        out = torch.empty((T, H, D_V), dtype=o_latent.dtype, device=o_latent.device)
    _bf16_tensor(out, (T, H, D_V), "out")
    mla_project_out(make_proj_params(tokens=T, num_heads=H), o_latent.data_ptr(), w_uv.data_ptr(), out.data_ptr(),
                    torch.cuda.current_stream(o_latent.device).cuda_stream)
    return out


def mla_expand_kv(params: PrefillParams, kv_ptr: int, block_table_ptr: int, t0: int, ntok: int, w_uk_ptr: int,
                  w_uv_ptr: int, k_ptr: int, vt_ptr: int, stream: int = 0) -> None:
    _check("mla_expand_kv", load_library().mla_expand_kv(
        ctypes.byref(params), kv_ptr or None, block_table_ptr or None, t0, ntok, w_uk_ptr or None, w_uv_ptr or None,
        k_ptr or None, vt_ptr or None, stream or None))


def mla_prefill_attention(params: PrefillParams, q_ptr: int, k_ptr: int, vt_ptr: int, t0: int, ntok: int,
                          out_ptr: int, lse_ptr: int, stream: int = 0) -> None:
    _check("mla_prefill_attention", load_library().mla_prefill_attention(
        ctypes.byref(params), q_ptr or None, k_ptr or None, vt_ptr or None, t0, ntok, out_ptr or None,
        lse_ptr or None, stream or None))


def mla_lse_merge(rows: int, nparts: int, parts_ptr: int, lparts_ptr: int, out_ptr: int, lse_ptr: int,
                  stream: int = 0) -> None:
    _check("mla_lse_merge", load_library().mla_lse_merge(
        rows, nparts, parts_ptr or None, lparts_ptr or None, out_ptr or None, lse_ptr or None, stream or None))


def mla_prefill_workspace_size(params: PrefillParams) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_prefill_workspace_size", load_library().mla_prefill_workspace_size(ctypes.byref(params),
                                                                                   ctypes.byref(n)))
    return n.value


def mla_chunked_prefill(params: PrefillParams, q_ptr: int, kv_ptr: int, block_table_ptr: int, w_uk_ptr: int,
                        w_uv_ptr: int, workspace_ptr: int, workspace_bytes: int, out_ptr: int, lse_ptr: int,
                        stream: int = 0) -> None:
    _check("mla_chunked_prefill", load_library().mla_chunked_prefill(
        ctypes.byref(params), q_ptr or None, kv_ptr or None, block_table_ptr or None, w_uk_ptr or None,
        w_uv_ptr or None, workspace_ptr or None, workspace_bytes, out_ptr or None, lse_ptr or None, stream or None))


class MlaPrefill:
    """The expand path for one request's new tokens on torch device tensors.

    q: bf16 [n, H, 192]; kv: the bf16 paged cache [P, 64, 576]; block_table: int32 row of the
    request; w_uk, w_uv: bf16 [H, 128, 512].  The workspace is allocated once here.
    """

    def __init__(self, *, num_heads, num_new, seqlen, num_pages, max_blocks, chunk_tokens=4096,
                 softmax_scale=1.0 / math.sqrt(D_NOPE + D_ROPE), device="cuda"):
        import torch
        self.params = make_prefill_params(num_heads=num_heads, num_new=num_new, seqlen=seqlen, num_pages=num_pages,
                                          max_blocks=max_blocks, chunk_tokens=chunk_tokens,
                                          softmax_scale=softmax_scale)
        self.ws_bytes = mla_prefill_workspace_size(self.params)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def __call__(self, q, kv, block_table, w_uk, w_uv, out=None, lse=None):
        import torch
        p = self.params
        n, H = p.num_new, p.num_heads
        _bf16_tensor(q, (n, H, D_NOPE + D_ROPE), "q")
        _bf16_tensor(w_uk, (H, D_NOPE, D_LATENT), "w_uk")
        _bf16_tensor(w_uv, (H, D_V, D_LATENT), "w_uv")
        if kv.element_size() != 2 or not kv.is_contiguous() or tuple(kv.shape[1:]) != (64, D_LATENT + D_ROPE):
            raise ValueError(f"kv: expected a contiguous 16-bit [P, 64, 576] cache, got {tuple(kv.shape)}")
        if block_table.dtype != torch.int32 or block_table.numel() < p.max_blocks or not block_table.is_contiguous():
            raise ValueError("block_table: expected a contiguous int32 row of max_blocks entries")
        if out is None:
            out = torch.empty((n, H, D_V), dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty((n, H), dtype=torch.float32, device=q.device)
        mla_chunked_prefill(p, q.data_ptr(), kv.data_ptr(), block_table.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                            self.workspace.data_ptr(), self.ws_bytes, out.data_ptr(), lse.data_ptr(),
                            torch.cuda.current_stream(q.device).cuda_stream)
        return out, lse


def _resolve_device(device):
    """torch.device with the index filled in ("cuda" -> the current HIP device)."""
    import torch
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    return dev


def check_decode_inputs(params: DecodeParams, device, q, kv_cache, block_table, seqlens, kv_scale=None) -> None:
    """Raise ValueError unless the tensors match what mla_decode_fwd reads for these parameters:
    q a contiguous 16-bit [B, s_q, H, 576]; kv_cache a contiguous [num_pages, 64, 576] of 16-bit values (bf16)
    or bytes (E4M3FN codes); kv_scale a contiguous float32 [num_pages, 64] exactly when the cache is FP8;
    block_table a contiguous int32 [B, max_blocks_per_seq]; seqlens a contiguous int32 [B]; all on `device`.
    The kernels index these buffers by the parameters alone, so a smaller or differently typed tensor would be
    read out of bounds."""
    import torch
    p = params
    B, s_q, H = p.batch, p.seqlen_q, p.num_heads
    fp8 = p.kv_dtype == MLA_KV_FP8_E4M3FN

    def need(cond, msg):
        if not cond:
            raise ValueError(msg)

    dev = _resolve_device(device)

    def on_dev(x, name):
        need(x.device == dev, f"{name}: on {x.device}, expected {dev}")
        need(x.is_contiguous(), f"{name}: must be contiguous")

    need(tuple(q.shape) == (B, s_q, H, HEAD_DIM_QK) and q.element_size() == 2,
         f"q: expected a 16-bit [{B}, {s_q}, {H}, {HEAD_DIM_QK}] tensor, got {q.dtype} {tuple(q.shape)}")
    on_dev(q, "q")
    kv_shape = (p.num_pages, PAGE_SIZE, HEAD_DIM_QK)
    if fp8:
        need(tuple(kv_cache.shape) == kv_shape and kv_cache.element_size() == 1,
             f"kv_cache: expected 1-byte E4M3FN codes of shape {kv_shape}, got {kv_cache.dtype} {tuple(kv_cache.shape)}")
        need(kv_scale is not None, "kv_scale: required for an FP8 cache")
        need(kv_scale.dtype == torch.float32 and tuple(kv_scale.shape) == (p.num_pages, PAGE_SIZE),
             f"kv_scale: expected float32 [{p.num_pages}, {PAGE_SIZE}], got {kv_scale.dtype} {tuple(kv_scale.shape)}")
        on_dev(kv_scale, "kv_scale")
    else:
        need(tuple(kv_cache.shape) == kv_shape and kv_cache.element_size() == 2,
             f"kv_cache: expected 16-bit bf16 values of shape {kv_shape}, got {kv_cache.dtype} {tuple(kv_cache.shape)}")
        need(kv_scale is None, "kv_scale: only an FP8 cache takes scales")
    on_dev(kv_cache, "kv_cache")
    need(block_table.dtype == torch.int32 and tuple(block_table.shape) == (B, p.max_blocks_per_seq),
         f"block_table: expected int32 [{B}, {p.max_blocks_per_seq}], got {block_table.dtype} {tuple(block_table.shape)}")
    on_dev(block_table, "block_table")
    need(seqlens.dtype == torch.int32 and tuple(seqlens.shape) == (B,),
         f"seqlens: expected int32 [{B}], got {seqlens.dtype} {tuple(seqlens.shape)}")
    on_dev(seqlens, "seqlens")


class MlaDecode:
    """One decode configuration bound to torch tensors on the current HIP device.

    ``plan(seqlens)`` runs the split plan; ``__call__`` runs decode + combine and
    returns (out bf16 [B, s_q, H, 512], lse fp32 [B, s_q, H]).  Buffers are
    allocated once, here, by torch; the library allocates nothing.
    """

    def __init__(self, *, batch, seqlen_q, num_heads, num_pages, max_blocks_per_seq, kv_dtype=MLA_KV_BF16,
                 causal=False, softmax_scale=SOFTMAX_SCALE, num_workgroups=0, fp8_path=MLA_FP8_PATH_EXACT,
                 device="cuda", debug=None):
        import torch
        self.torch = torch
        # Debug mode: before each decode, synchronous checks of the device-side values the kernels otherwise
        # only clamp and flag (every length in [seqlen_q, max_blocks_per_seq * 64], every block-table entry a
        # request uses in [0, num_pages)); after decode + combine, any workspace flag raises MlaDeviceError.
        # Each check synchronises the stream: for testing and bring-up, not for timing.
        self.debug = debug_from_env() if debug is None else bool(debug)
        self.params = make_params(batch=batch, seqlen_q=seqlen_q, num_heads=num_heads, num_pages=num_pages,
                                  max_blocks_per_seq=max_blocks_per_seq, kv_dtype=kv_dtype, causal=causal,
                                  softmax_scale=softmax_scale, num_workgroups=num_workgroups, fp8_path=fp8_path)
        self.device = _resolve_device(device)
        self.workspace_bytes = mla_get_workspace(self.params)
        # 256-byte aligned: the caching allocator hands out 512-byte aligned blocks.
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)
        self.out = torch.empty((batch, seqlen_q, num_heads, HEAD_DIM_V), dtype=torch.bfloat16, device=self.device)
        self.lse = torch.empty((batch, seqlen_q, num_heads), dtype=torch.float32, device=self.device)

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def plan(self, seqlens) -> None:
        import torch
        if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (self.params.batch,) or \
                seqlens.device != self.device or not seqlens.is_contiguous():
            raise ValueError(f"seqlens: expected a contiguous int32 [{self.params.batch}] tensor on {self.device}")
        mla_get_workspace(self.params, seqlens.data_ptr(), self.workspace.data_ptr(), self.workspace_bytes,
                          self._stream())

    def check_device_values(self, block_table, seqlens) -> None:
        """The debug mode's synchronous checks (raises MlaDeviceError)."""
        p = self.params
        sl = seqlens.cpu()
        lo, hi = p.seqlen_q, p.max_blocks_per_seq * PAGE_SIZE
        bad = ((sl < lo) | (sl > hi)).nonzero().flatten().tolist()
        if bad:
            b = bad[0]
            raise MlaDeviceError(f"seqlens[{b}] = {int(sl[b])} is outside [{lo}, {hi}]", MLA_FLAG_SEQLEN_CLAMPED)
        import torch
        bt = block_table.cpu()
        used = torch.arange(p.max_blocks_per_seq)[None, :] < ((sl + PAGE_SIZE - 1) // PAGE_SIZE)[:, None]
        bad = (used & ((bt < 0) | (bt >= p.num_pages))).nonzero()
        if len(bad):
            b, j = int(bad[0, 0]), int(bad[0, 1])
            raise MlaDeviceError(f"block_table[{b}][{j}] = {int(bt[b, j])} is outside [0, {p.num_pages})",
                                 MLA_FLAG_BAD_BLOCK)

    def raise_on_flags(self) -> None:
        """Debug mode: raise MlaDeviceError if a kernel has set a workspace flag."""
        f = self.flags()
        if f:
            raise MlaDeviceError(f"decode reported: {describe_flags(f)} (flags 0x{f:x})", f)

    def decode(self, q, kv_cache, block_table, seqlens, kv_scale=None) -> None:
        check_decode_inputs(self.params, self.device, q, kv_cache, block_table, seqlens, kv_scale)
        if self.debug:
            self.check_device_values(block_table, seqlens)
        mla_decode_fwd(self.params, q.data_ptr(), kv_cache.data_ptr(), 0 if kv_scale is None else kv_scale.data_ptr(),
                       block_table.data_ptr(), seqlens.data_ptr(), self.workspace.data_ptr(), self.workspace_bytes,
                       self.out.data_ptr(), self.lse.data_ptr(), self._stream())

    def combine(self) -> None:
        mla_splitkv_combine(self.params, self.workspace.data_ptr(), self.workspace_bytes, self.out.data_ptr(),
                            self.lse.data_ptr(), self._stream())

    def __call__(self, q, kv_cache, block_table, seqlens, kv_scale=None, plan=True):
        if plan:
            self.plan(seqlens)
        self.decode(q, kv_cache, block_table, seqlens, kv_scale)
        self.combine()
        if self.debug:
            self.raise_on_flags()
        return self.out, self.lse

    def flags(self) -> int:
        return mla_workspace_flags(self.workspace.data_ptr(), self._stream())
