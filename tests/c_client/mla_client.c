/* mla_client.c -- a plain C program driving libmla_decode.so through its C ABI
 * (include/mla_decode.h): device buffers from the HIP runtime, the split plan,
 * the attention kernel and the split-KV merge, then every output row checked
 * against the fp64 oracle (oracle/mla_oracle.c, linked as liboracle.so).  No
 * Python and no torch: the library is used the way a C or C++ serving engine
 * would use it.  Exit status 0 when every row is within the tolerances. */
#define __HIP_PLATFORM_AMD__
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla_decode.h"

/* The oracle's entry point and shape record (declared in oracle/mla_oracle.c). */
typedef struct {
  int32_t batch, seqlen_q, num_heads, d_latent, d_rope, page_size, num_pages, max_blocks, causal, q_dtype, kv_dtype;
  float softmax_scale;
} oracle_shape;
int oracle_mla_attend(const oracle_shape* s, const void* q, const void* cache, const float* kv_scale,
                      const int32_t* block_table, const int32_t* seqlens, const int32_t* t_begin,
                      const int32_t* t_end, const int64_t* rows, int64_t nrows, double* out, double* lse);

#define CHECK_HIP(x)                                                          \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 2;                                                               \
    }                                                                         \
  } while (0)
#define CHECK_MLA(x)                                                          \
  do {                                                                        \
    int s_ = (x);                                                             \
    if (s_ != MLA_OK) {                                                       \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, mla_status_string(s_)); \
      return 2;                                                               \
    }                                                                         \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float uniform_pm1(void) { /* xorshift64*, top 24 bits -> [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  const uint64_t r = rng_state * 0x2545F4914F6CDD1Dull;
  return (float)(r >> 40) / (float)(1u << 23) - 1.0f;
}
static uint16_t to_bf16(float x) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  enum { B = 3, SQ = 2, H = 16, D = 576, DV = 512, PAGE = 64, MAXB = 12 };
  const int32_t seqlens[B] = {100, 2, 700};
  const float scale = 1.0f / sqrtf(192.0f);
  int32_t bt[B][MAXB];
  int npages = 0;
  for (int b = 0; b < B; b++) npages += (seqlens[b] + PAGE - 1) / PAGE;
  /* pages handed out in reverse order: a scattered physical layout */
  int next = npages - 1;
  for (int b = 0; b < B; b++)
    for (int j = 0; j < MAXB; j++) bt[b][j] = j < (seqlens[b] + PAGE - 1) / PAGE ? next-- : -1;
  const size_t nq = (size_t)B * SQ * H * D, nkv = (size_t)npages * PAGE * D, nrows = (size_t)B * SQ * H;
  uint16_t* q = malloc(nq * 2);
  uint16_t* kv = malloc(nkv * 2);
  uint16_t* out = malloc(nrows * DV * 2);
  float* lse = malloc(nrows * 4);
  double* ref = malloc(nrows * DV * sizeof(double));
  double* ref_lse = malloc(nrows * sizeof(double));
  if (!q || !kv || !out || !lse || !ref || !ref_lse) return 2;
  for (size_t i = 0; i < nq; i++) q[i] = to_bf16(2.0f * uniform_pm1());
  for (size_t i = 0; i < nkv; i++) kv[i] = to_bf16(2.0f * uniform_pm1());

  mla_decode_params p = {0};
  p.batch = B;
  p.seqlen_q = SQ;
  p.num_heads = H;
  p.head_dim_qk = D;
  p.head_dim_v = DV;
  p.page_size = PAGE;
  p.num_pages = npages;
  p.max_blocks_per_seq = MAXB;
  p.kv_dtype = MLA_KV_BF16;
  p.causal = 1;
  p.softmax_scale = scale;
  p.num_workgroups = 7; /* a small workgroup count: the long request is split and merged */
  p.fp8_path = MLA_FP8_PATH_EXACT;

  void *d_q, *d_kv, *d_bt, *d_sl, *d_out, *d_lse, *d_ws;
  size_t ws_bytes = 0;
  CHECK_MLA(mla_get_workspace(&p, NULL, NULL, &ws_bytes, NULL));
  CHECK_HIP(hipMalloc(&d_q, nq * 2));
  CHECK_HIP(hipMalloc(&d_kv, nkv * 2));
  CHECK_HIP(hipMalloc(&d_bt, sizeof(bt)));
  CHECK_HIP(hipMalloc(&d_sl, sizeof(seqlens)));
  CHECK_HIP(hipMalloc(&d_out, nrows * DV * 2));
  CHECK_HIP(hipMalloc(&d_lse, nrows * 4));
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_HIP(hipMemcpy(d_q, q, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_kv, kv, nkv * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_bt, bt, sizeof(bt), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_sl, seqlens, sizeof(seqlens), hipMemcpyHostToDevice));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  CHECK_MLA(mla_get_workspace(&p, d_sl, d_ws, &ws_bytes, stream));
  CHECK_MLA(mla_decode_fwd(&p, d_q, d_kv, NULL, d_bt, d_sl, d_ws, ws_bytes, d_out, d_lse, stream));
  CHECK_MLA(mla_splitkv_combine(&p, d_ws, ws_bytes, d_out, d_lse, stream));
  uint32_t flags = 0;
  CHECK_MLA(mla_workspace_flags(d_ws, &flags, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(out, d_out, nrows * DV * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse, d_lse, nrows * 4, hipMemcpyDeviceToHost));

  const oracle_shape s = {B, SQ, H, DV, D - DV, PAGE, npages, MAXB, 1, 0, 0, scale};
  const int32_t t_begin[B] = {0, 0, 0};
  if (oracle_mla_attend(&s, q, kv, NULL, &bt[0][0], seqlens, t_begin, seqlens, NULL, (int64_t)nrows, ref, ref_lse))
    return 2;
  double max_abs = 0, num = 0, den = 0, lse_err = 0;
  for (size_t r = 0; r < nrows; r++) {
    for (int d = 0; d < DV; d++) {
      const double g = from_bf16(out[r * DV + d]), e = ref[r * DV + d];
      if (!(fabs(g - e) <= max_abs)) max_abs = fabs(g - e); /* NaN-safe: a NaN makes max_abs NaN */
      num += (g - e) * (g - e);
      den += e * e;
    }
    const double le = fabs((double)lse[r] - ref_lse[r]);
    if (!(le <= lse_err)) lse_err = le;
  }
  const double rel = sqrt(num / den);
  printf("mla_client: %zu rows, workspace %zu bytes, flags %u: out max-abs %.3e rel-L2 %.3e, lse max-abs %.3e\n",
         nrows, ws_bytes, flags, max_abs, rel, lse_err);
  const int ok = flags == 0 && max_abs <= 2e-2 && rel <= 5e-3 && lse_err <= 1e-3;
  hipFree(d_q);
  hipFree(d_kv);
  hipFree(d_bt);
  hipFree(d_sl);
  hipFree(d_out);
  hipFree(d_lse);
  hipFree(d_ws);
  hipStreamDestroy(stream);
  free(q);
  free(kv);
  free(out);
  free(lse);
  free(ref);
  free(ref_lse);
  return ok ? 0 : 1;
}
