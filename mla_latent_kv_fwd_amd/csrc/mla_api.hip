// mla_api.hip -- the C ABI of libmla_decode.so (declared in include/mla_decode.h
// and include/mla_proj.h):
// argument validation, workspace sizing and kernel launches.  No device memory
// is allocated here; the caller owns every buffer.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>

#define MLA_HD __host__ __device__
#include "mla_decode.h"
#include "mla_proj.h"
#include "mla_prefill.h"
#include "mla_launch.h"
#include "mla_workspace.h"

namespace {

using namespace mla;

constexpr int kMaxDevices = 64;

// Compute-unit count per device, queried once.
int device_cu_count(int dev) {
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return -1;
  std::call_once(once[dev], [dev] {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = -1;
    cus[dev] = v;
  });
  return cus[dev];
}

int validate(const mla_decode_params* p) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->batch > kMaxBatch) return MLA_ERR_INVALID_ARG;
  if (p->seqlen_q < 1 || p->num_heads < 1 || p->num_pages < 1 || p->max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (p->num_workgroups < 0) return MLA_ERR_INVALID_ARG;
  if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (p->fp8_path != MLA_FP8_PATH_EXACT && p->fp8_path != MLA_FP8_PATH_MFMA) return MLA_ERR_INVALID_ARG;
  if (p->fp8_path == MLA_FP8_PATH_MFMA && p->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (p->head_dim_qk != kHeadDimQK || p->head_dim_v != kHeadDimV || p->page_size != kPageSize)
    return MLA_ERR_UNSUPPORTED;
  if (p->seqlen_q > kMaxSeqlenQ || p->num_heads > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  // page positions and token counts are int32 inside the kernels
  if ((int64_t)p->batch * p->max_blocks_per_seq >= ((int64_t)1 << 31) / kPageSize) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_pages >= ((int64_t)1 << 31) / kPageSize) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// Number of stretches (persistent workgroups per row block).  Deterministic in p
// and the device, so the size query, the plan and the decode all agree.
int resolve_nwg(const mla_decode_params* p, int* nwg) {
  const int nrb = row_blocks(p->seqlen_q * p->num_heads);
  int want = p->num_workgroups;
  if (want == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    const int cus = device_cu_count(dev);
    if (cus <= 0) return MLA_ERR_HIP;
    want = cus / nrb > 0 ? cus / nrb : 1;
  }
  const int64_t max_pages = (int64_t)p->batch * p->max_blocks_per_seq;
  int64_t v = want;
  if (v > max_pages) v = max_pages;
  if (v > kMaxStretches) v = kMaxStretches;
  *nwg = (int)(v < 1 ? 1 : v);
  return MLA_OK;
}

constexpr int kMaxProjTokens = 65536;

int validate_proj(const mla_proj_params* p) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->tokens < 1 || p->tokens > kMaxProjTokens || p->num_heads < 1) return MLA_ERR_INVALID_ARG;
  if (p->num_heads > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  if (p->d_nope != 128 || p->d_rope != 64 || p->d_latent != 512 || p->d_v != 128) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

bool misaligned16(const void* ptr) { return ((uintptr_t)ptr & 15) != 0; }

constexpr int kMaxPrefillNew = 65536;
constexpr int kMaxChunkTokens = 65536;
constexpr int kMaxMergeParts = 4096;

int validate_prefill(const mla_prefill_params* p) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->num_heads < 1 || p->num_new < 1 || p->num_new > kMaxPrefillNew || p->seqlen < p->num_new)
    return MLA_ERR_INVALID_ARG;
  if (p->num_pages < 1 || p->max_blocks < 1) return MLA_ERR_INVALID_ARG;
  if ((int64_t)p->max_blocks * kPageSize >= ((int64_t)1 << 31)) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)p->seqlen > (int64_t)p->max_blocks * kPageSize) return MLA_ERR_INVALID_ARG;
  if (p->chunk_tokens < 64 || p->chunk_tokens > kMaxChunkTokens || p->chunk_tokens % 64) return MLA_ERR_INVALID_ARG;
  if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (p->num_heads > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  if (p->d_nope != 128 || p->d_rope != 64 || p->d_latent != 512 || p->d_v != 128) return MLA_ERR_UNSUPPORTED;
  if ((p->seqlen + p->chunk_tokens - 1) / p->chunk_tokens > kMaxMergeParts) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunked-prefill workspace: one expanded K and V^T chunk, then the fp32 partials and
// LSEs of every chunk.
struct PrefillLayout {
  size_t k, vt, parts, lparts, total;
  int nchunks;
};
PrefillLayout prefill_layout(const mla_prefill_params* p) {
  PrefillLayout l;
  const size_t H = p->num_heads, Tc = p->chunk_tokens, rows = (size_t)p->num_new * H;
  l.nchunks = (p->seqlen + p->chunk_tokens - 1) / p->chunk_tokens;
  l.k = 0;
  l.vt = align256(l.k + H * Tc * 192 * 2);
  l.parts = align256(l.vt + H * 128 * Tc * 2);
  l.lparts = align256(l.parts + (size_t)l.nchunks * rows * 128 * 4);
  l.total = align256(l.lparts + (size_t)l.nchunks * rows * 4);
  return l;
}

// The no-allocation path's workspace: one fixed array per GPU, in the code
// object's zero-initialised data.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

void* scratch_address(int dev) {
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) ptr = nullptr;
    addr[dev] = ptr;
  });
  return addr[dev];
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_SCRATCH_TOO_SMALL: return "step needs more than the fixed no-allocation scratch";
    default: return "unknown status";
  }
}

int mla_get_workspace(const mla_decode_params* p, const int32_t* seqlens, void* workspace, size_t* workspace_bytes,
                      void* stream) {
  int st = validate(p);
  if (st != MLA_OK) return st;
  if (!workspace_bytes) return MLA_ERR_INVALID_ARG;
  int nwg = 0;
  if ((st = resolve_nwg(p, &nwg)) != MLA_OK) return st;
  const int rows = p->seqlen_q * p->num_heads;
  const Layout lay = make_layout(p->batch, rows, nwg);
  if (!workspace) {
    *workspace_bytes = lay.total;
    return MLA_OK;
  }
  if (!seqlens || ((uintptr_t)workspace & 255)) return MLA_ERR_INVALID_ARG;
  if (*workspace_bytes < lay.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (launch_plan(seqlens, workspace, lay, p->batch, p->seqlen_q, rows, nwg, p->max_blocks_per_seq,
                  (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_decode_fwd(const mla_decode_params* p, const void* q, const void* kv_cache, const float* kv_scale,
                   const int32_t* block_table, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                   void* out, float* lse, void* stream) {
  int st = validate(p);
  if (st != MLA_OK) return st;
  if (!q || !kv_cache || !block_table || !seqlens || !workspace || !out || !lse) return MLA_ERR_INVALID_ARG;
  if ((p->kv_dtype == MLA_KV_FP8_E4M3FN) != (kv_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)q & 15) || ((uintptr_t)kv_cache & 15) || ((uintptr_t)out & 7) || ((uintptr_t)workspace & 255) ||
      ((uintptr_t)kv_scale & 15))
    return MLA_ERR_INVALID_ARG;
  int nwg = 0;
  if ((st = resolve_nwg(p, &nwg)) != MLA_OK) return st;
  const int rows = p->seqlen_q * p->num_heads;
  const Layout lay = make_layout(p->batch, rows, nwg);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = kv_cache;
  a.kv_scale = kv_scale;
  a.block_table = block_table;
  a.ws = static_cast<char*>(workspace);
  a.lay = lay;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.batch = p->batch;
  a.seqlen_q = p->seqlen_q;
  a.num_heads = p->num_heads;
  a.rows = rows;
  a.nrb = row_blocks(rows);
  a.nwg = nwg;
  a.num_pages = p->num_pages;
  a.max_blocks = p->max_blocks_per_seq;
  a.causal = p->causal ? 1 : 0;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  const hipError_t e = p->fp8_path == MLA_FP8_PATH_MFMA
                           ? launch_decode_fp8_mfma(a, (hipStream_t)stream)
                           : launch_decode(a, p->kv_dtype == MLA_KV_FP8_E4M3FN, (hipStream_t)stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_decode_noalloc(const mla_decode_params* p, const void* q, const void* kv_cache, const float* kv_scale,
                       const int32_t* block_table, const int32_t* seqlens, void* out, float* lse, void* stream) {
  int st = validate(p);
  if (st != MLA_OK) return st;
  if (!q || !kv_cache || !block_table || !seqlens || !out || !lse) return MLA_ERR_INVALID_ARG;
  int nwg = 0;
  if ((st = resolve_nwg(p, &nwg)) != MLA_OK) return st;
  const Layout lay = make_layout(p->batch, p->seqlen_q * p->num_heads, nwg);
  if (lay.total > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH_TOO_SMALL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return MLA_ERR_HIP;
  // The plan writes every plan entry and header field the decode reads, and the
  // decode writes every partial the combine reads: nothing needs clearing.
  size_t nbytes = lay.total;
  if ((st = mla_get_workspace(p, seqlens, ws, &nbytes, stream)) != MLA_OK) return st;
  if ((st = mla_decode_fwd(p, q, kv_cache, kv_scale, block_table, seqlens, ws, lay.total, out, lse, stream)) !=
      MLA_OK)
    return st;
  return mla_splitkv_combine(p, ws, lay.total, out, lse, stream);
}

int mla_splitkv_combine(const mla_decode_params* p, const void* workspace, size_t workspace_bytes, void* out,
                        float* lse, void* stream) {
  int st = validate(p);
  if (st != MLA_OK) return st;
  if (!workspace || !out || !lse || ((uintptr_t)workspace & 255) || ((uintptr_t)out & 7)) return MLA_ERR_INVALID_ARG;
  int nwg = 0;
  if ((st = resolve_nwg(p, &nwg)) != MLA_OK) return st;
  const int rows = p->seqlen_q * p->num_heads;
  const Layout lay = make_layout(p->batch, rows, nwg);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (launch_combine(static_cast<const char*>(workspace), lay, p->batch, rows, nwg, p->max_blocks_per_seq,
                     static_cast<uint16_t*>(out), lse, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_absorb_q(const mla_proj_params* p, const void* q_nope, const void* q_rope, const void* w_uk, void* q_tilde,
                 void* stream) {
  const int st = validate_proj(p);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_rope || !w_uk || !q_tilde) return MLA_ERR_INVALID_ARG;
  if (misaligned16(q_nope) || misaligned16(q_rope) || misaligned16(w_uk) || misaligned16(q_tilde))
    return MLA_ERR_INVALID_ARG;
  if (launch_absorb_q(static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
                      static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_tilde), p->tokens, p->num_heads,
                      (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_project_out(const mla_proj_params* p, const void* o_latent, const void* w_uv, void* out, void* stream) {
  const int st = validate_proj(p);
  if (st != MLA_OK) return st;
  if (!o_latent || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (misaligned16(o_latent) || misaligned16(w_uv) || misaligned16(out)) return MLA_ERR_INVALID_ARG;
  if (launch_project_out(static_cast<const uint16_t*>(o_latent), static_cast<const uint16_t*>(w_uv),
                         static_cast<uint16_t*>(out), p->tokens, p->num_heads, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_workspace_flags(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return MLA_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  Header h;
  if (hipMemcpy(&h, workspace, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  *flags = h.magic == kMagic ? h.flags : (uint32_t)MLA_FLAG_BAD_PLAN;   // never planned
  return MLA_OK;
}

int mla_expand_kv(const mla_prefill_params* p, const void* kv_cache, const int32_t* block_table, int32_t t0,
                  int32_t ntok, const void* w_uk, const void* w_uv, void* k_out, void* vt_out, void* stream) {
  const int st = validate_prefill(p);
  if (st != MLA_OK) return st;
  if (!kv_cache || !block_table || !w_uk || !w_uv || !k_out || !vt_out) return MLA_ERR_INVALID_ARG;
  if (misaligned16(kv_cache) || misaligned16(w_uk) || misaligned16(w_uv) || misaligned16(k_out) || misaligned16(vt_out))
    return MLA_ERR_INVALID_ARG;
  if (t0 < 0 || ntok < 1 || ntok > kMaxChunkTokens || (int64_t)t0 + ntok > p->seqlen) return MLA_ERR_INVALID_ARG;
  if (launch_expand_kv(static_cast<const uint16_t*>(kv_cache), block_table, t0, ntok, p->num_pages,
                       static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
                       static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(vt_out), p->num_heads,
                       (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_prefill_attention(const mla_prefill_params* p, const void* q, const void* k, const void* vt, int32_t t0,
                          int32_t ntok, float* out, float* lse, void* stream) {
  const int st = validate_prefill(p);
  if (st != MLA_OK) return st;
  if (!q || !k || !vt || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (misaligned16(q) || misaligned16(k) || misaligned16(vt) || misaligned16(out) || ((uintptr_t)lse & 3))
    return MLA_ERR_INVALID_ARG;
  if (t0 < 0 || ntok < 1 || ntok > kMaxChunkTokens || (int64_t)t0 + ntok > p->seqlen) return MLA_ERR_INVALID_ARG;
  if (launch_prefill_attention(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                               static_cast<const uint16_t*>(vt), t0, ntok, p->num_new, p->seqlen, p->num_heads,
                               p->softmax_scale, out, lse, nullptr, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_lse_merge(int32_t rows, int32_t nparts, const float* out_parts, const float* lse_parts, void* out, float* lse,
                  void* stream) {
  if (rows < 1 || rows > (1 << 24) || nparts < 1 || nparts > kMaxMergeParts) return MLA_ERR_INVALID_ARG;
  if (!out_parts || !lse_parts || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (misaligned16(out_parts) || misaligned16(out) || ((uintptr_t)lse_parts & 3) || ((uintptr_t)lse & 3))
    return MLA_ERR_INVALID_ARG;
  if (launch_lse_merge(rows, nparts, out_parts, lse_parts, static_cast<uint16_t*>(out), lse, (hipStream_t)stream) !=
      hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_prefill_workspace_size(const mla_prefill_params* p, size_t* bytes) {
  const int st = validate_prefill(p);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  *bytes = prefill_layout(p).total;
  return MLA_OK;
}

int mla_chunked_prefill(const mla_prefill_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                        const void* w_uk, const void* w_uv, void* workspace, size_t workspace_bytes, void* out,
                        float* lse, void* stream) {
  const int st = validate_prefill(p);
  if (st != MLA_OK) return st;
  if (!q || !kv_cache || !block_table || !w_uk || !w_uv || !workspace || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (misaligned16(q) || misaligned16(kv_cache) || misaligned16(w_uk) || misaligned16(w_uv) || misaligned16(out) ||
      ((uintptr_t)workspace & 255) || ((uintptr_t)lse & 3))
    return MLA_ERR_INVALID_ARG;
  const PrefillLayout l = prefill_layout(p);
  if (workspace_bytes < l.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  uint16_t* kbuf = reinterpret_cast<uint16_t*>(ws + l.k);
  uint16_t* vtbuf = reinterpret_cast<uint16_t*>(ws + l.vt);
  float* parts = reinterpret_cast<float*>(ws + l.parts);
  float* lparts = reinterpret_cast<float*>(ws + l.lparts);
  const size_t rows = (size_t)p->num_new * p->num_heads;
  const hipStream_t s = (hipStream_t)stream;
  // One chunk: the attention writes the final bf16 rows and LSEs itself (the merge
  // of a single part is the identity up to that rounding).
  const bool single = l.nchunks == 1;
  for (int j = 0; j < l.nchunks; j++) {
    const int t0 = j * p->chunk_tokens;
    const int ntok = p->seqlen - t0 < p->chunk_tokens ? p->seqlen - t0 : p->chunk_tokens;
    if (launch_expand_kv(static_cast<const uint16_t*>(kv_cache), block_table, t0, ntok, p->num_pages,
                         static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv), kbuf, vtbuf,
                         p->num_heads, s) != hipSuccess)
      return MLA_ERR_HIP;
    if (launch_prefill_attention(static_cast<const uint16_t*>(q), kbuf, vtbuf, t0, ntok, p->num_new, p->seqlen,
                                 p->num_heads, p->softmax_scale, single ? nullptr : parts + (size_t)j * rows * 128,
                                 single ? lse : lparts + (size_t)j * rows,
                                 single ? static_cast<uint16_t*>(out) : nullptr, s) != hipSuccess)
      return MLA_ERR_HIP;
  }
  if (!single &&
      launch_lse_merge((int)rows, l.nchunks, parts, lparts, static_cast<uint16_t*>(out), lse, s) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
