// mla_launch.h -- host-side launchers of the library's kernels.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_workspace.h"

namespace mla {

// Everything the decode kernel reads, passed by value.
struct DecodeArgs {
  const uint16_t* q;          // bf16 [B][s_q][H][576]
  const void* kv;             // [P][64][576] bf16 or E4M3FN
  const float* kv_scale;      // [P][64] (FP8 only)
  const int32_t* block_table; // [B][max_blocks]
  char* ws;
  Layout lay;
  uint16_t* out;              // bf16 [B][s_q][H][512]
  float* lse;                 // [B][s_q][H]
  int batch, seqlen_q, num_heads, rows, nrb, nwg, num_pages, max_blocks, causal;
  float scale_log2;           // softmax_scale * log2(e)
};

hipError_t launch_plan(const int32_t* seqlens, void* ws, const Layout& lay, int batch, int seqlen_q, int rows,
                       int nwg, int max_blocks, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_decode_fp8_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine(const char* ws, const Layout& lay, int batch, int rows, int nwg, int max_blocks,
                          uint16_t* out, float* lse, hipStream_t stream);
hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, uint16_t* q_tilde,
                           int T, int H, hipStream_t stream);
hipError_t launch_project_out(const uint16_t* o_latent, const uint16_t* w_uv, uint16_t* out, int T, int H,
                              hipStream_t stream);

// Expand path (mla_prefill.hip).
hipError_t launch_expand_kv(const uint16_t* cache, const int32_t* block_table, int t0, int ntok, int num_pages,
                            const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* k_out, uint16_t* vt_out, int H,
                            hipStream_t stream);
// out16 non-null: the rows go out in bf16 to out16 (final output of a single-chunk
// call) instead of fp32 to out.
hipError_t launch_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int t0, int ntok, int n,
                                    int L, int H, float softmax_scale, float* out, float* lse, uint16_t* out16,
                                    hipStream_t stream);
hipError_t launch_lse_merge(int rows, int J, const float* parts, const float* lparts, uint16_t* out, float* lse,
                            hipStream_t stream);

}  // namespace mla
