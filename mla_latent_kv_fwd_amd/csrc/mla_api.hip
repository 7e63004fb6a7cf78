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

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
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
  if (launch_decode(a, p->kv_dtype == MLA_KV_FP8_E4M3FN, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
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
  if (launch_combine(static_cast<const char*>(workspace), lay, p->batch, rows, static_cast<uint16_t*>(out), lse,
                     (hipStream_t)stream) != hipSuccess)
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
  *flags = h.magic == kMagic ? h.flags : 0u;
  return MLA_OK;
}

}  // extern "C"
