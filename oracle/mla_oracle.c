/*
 * mla_oracle.c -- fp64 CPU reference for multi-head latent attention (MLA)
 * decode on the absorb path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the HIP
 * path.
 *
 * What is computed (sources are the pages' own sections):
 *
 *  - The score of a query row against cached token t is one dot product over
 *    the concatenated latent and RoPE parts: the content part q^N.(W_UK c)
 *    equals (W_UK^T q^N).c, so with the absorbed query q~ = [W_UK^T q^N ; q^R]
 *    and the cache row [c ; k^R] the score is q~.[c ; k^R]
 *    ("MLA inference: two computation paths and FlashMLA", section "Two
 *    equivalent paths", score equation and path two).
 *  - Logits are scaled by 1/sqrt(d_nope + d_rope) = 1/sqrt(192) at DeepSeek-V3
 *    shapes (same page, worked example; "FlashMLA: Fast Hopper Decoding ...",
 *    Architecture step 3).  The scale is an argument here.
 *  - Softmax over the visible cached tokens, then the weighted sum is taken in
 *    latent space: the value of token t is its latent c_t, i.e. the first
 *    d_latent numbers of the cache row (handbook page, path two: the weighted
 *    sum is in latent space and W_UV is applied afterwards).
 *  - The log-sum-exp of the scaled logits is returned with every output row so
 *    that partial results over disjoint token ranges can be merged (handbook
 *    page, "Which is faster", merge by LSE; "Decode attention becomes a compute
 *    problem", split-KV).
 *  - Paged cache: logical token t of request b lives in physical page
 *    block_table[b][t / page_size], slot t % page_size (handbook page, FlashMLA
 *    paragraph: paged KV with block size 64; FlashMLA guide, Architecture 1).
 *  - With several new tokens per request, seqlen counts the new tokens and new
 *    token i sees the keys up to and including itself: L - s_q + 1 + i keys
 *    (handbook page, FLOP script: its cached-token count already holds the
 *    new tokens, and its causal pair count is the sum of these key counts).
 *  - FP8 cache: OCP E4M3FN codes (1 sign, 4 exponent, 3 mantissa bits, max 448;
 *    "MLA and FP8 MoE Serving", section on FP8 formats) times a per-token fp32
 *    scale.
 *
 * Precision: every stored input is widened exactly to double (bf16 and
 * E4M3FN values are exactly representable), all arithmetic is in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1, ORACLE_BAD_BLOCK = -2, ORACLE_BAD_SEQLEN = -3, ORACLE_NOMEM = -4 };
enum { ORACLE_Q_BF16 = 0, ORACLE_Q_F64 = 1 };
enum { ORACLE_KV_BF16 = 0, ORACLE_KV_E4M3FN = 1 };

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3FN: exponent bias 7, no infinities, S.1111.111 is NaN,
 * exponent field 0 holds subnormals m/8 * 2^(1-7). */
double oracle_e4m3fn_to_f64(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, 1 - 7);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Shape and dtype description shared by the entry points below. */
typedef struct {
  int32_t batch;          /* B */
  int32_t seqlen_q;       /* s_q: new tokens per request */
  int32_t num_heads;      /* H */
  int32_t d_latent;       /* 512 at DeepSeek-V3 shapes; also the value width */
  int32_t d_rope;         /* 64 at DeepSeek-V3 shapes */
  int32_t page_size;      /* tokens per page */
  int32_t num_pages;      /* physical pages in the cache */
  int32_t max_blocks;     /* row stride of the block table */
  int32_t causal;         /* mask among the s_q new tokens */
  int32_t q_dtype;        /* ORACLE_Q_BF16 or ORACLE_Q_F64 */
  int32_t kv_dtype;       /* ORACLE_KV_BF16 or ORACLE_KV_E4M3FN */
  float softmax_scale;    /* the fp32 value the caller passes; widened exactly */
} oracle_shape;

static double q_value(const oracle_shape* s, const void* q, size_t idx) {
  if (s->q_dtype == ORACLE_Q_F64) return ((const double*)q)[idx];
  return oracle_bf16_to_f64(((const uint16_t*)q)[idx]);
}

/* Widen one cached token (all d_latent + d_rope numbers) of request b at
 * logical position t into kv[].  Returns 0, or ORACLE_BAD_BLOCK if the block
 * table points outside the cache. */
static int gather_token(const oracle_shape* s, const void* cache, const float* kv_scale,
                        const int32_t* block_table, int b, int t, double* kv) {
  const int D = s->d_latent + s->d_rope;
  const int32_t page = block_table[(size_t)b * s->max_blocks + t / s->page_size];
  const int slot = t % s->page_size;
  if (page < 0 || page >= s->num_pages) return ORACLE_BAD_BLOCK;
  const size_t row = ((size_t)page * s->page_size + slot) * (size_t)D;
  if (s->kv_dtype == ORACLE_KV_E4M3FN) {
    const double scale = (double)kv_scale[(size_t)page * s->page_size + slot];
    for (int d = 0; d < D; d++) kv[d] = oracle_e4m3fn_to_f64(((const uint8_t*)cache)[row + d]) * scale;
  } else {
    for (int d = 0; d < D; d++) kv[d] = oracle_bf16_to_f64(((const uint16_t*)cache)[row + d]);
  }
  return ORACLE_OK;
}

/* Number of cached tokens that new-token row i of a request of length L may
 * attend to. */
static int visible_keys(const oracle_shape* s, int L, int i) {
  return s->causal ? L - s->seqlen_q + 1 + i : L;
}

/*
 * Attention of the selected rows over the token window [t_begin[b], t_end[b])
 * of each request, clipped to the row's visible keys.  A full decode passes
 * t_begin = 0 and t_end = seqlens.  A row whose window is empty gets LSE = -inf
 * and a zero output (the neutral element of the merge below).
 *
 * q:      [B][s_q][H][d_latent + d_rope], bf16 bits or double
 * cache:  [num_pages][page_size][d_latent + d_rope], bf16 bits or E4M3FN codes
 * kv_scale: [num_pages][page_size] fp32, E4M3FN only
 * rows:   flat row ids ((b * s_q + i) * H + h); NULL means every row in order
 * out:    [nrows][d_latent]; lse: [nrows]
 */
int oracle_mla_attend(const oracle_shape* s, const void* q, const void* cache, const float* kv_scale,
                      const int32_t* block_table, const int32_t* seqlens, const int32_t* t_begin,
                      const int32_t* t_end, const int64_t* rows, int64_t nrows, double* out, double* lse) {
  if (!s || !q || !cache || !block_table || !seqlens || !out || !lse) return ORACLE_BAD_ARG;
  if (s->batch < 0 || s->seqlen_q < 1 || s->num_heads < 1 || s->d_latent < 1 || s->d_rope < 0 ||
      s->page_size < 1 || s->max_blocks < 0 || s->num_pages < 0)
    return ORACLE_BAD_ARG;
  if (s->kv_dtype == ORACLE_KV_E4M3FN && !kv_scale) return ORACLE_BAD_ARG;
  const int64_t total_rows = (int64_t)s->batch * s->seqlen_q * s->num_heads;
  if (!rows) nrows = total_rows;
  for (int b = 0; b < s->batch; b++) {
    const int L = seqlens[b];
    if (L < s->seqlen_q || (int64_t)L > (int64_t)s->max_blocks * s->page_size) return ORACLE_BAD_SEQLEN;
  }
  const int D = s->d_latent + s->d_rope;
  const int Dv = s->d_latent;
  int status = ORACLE_OK;

#pragma omp parallel
  {
    double* kv = (double*)malloc(sizeof(double) * (size_t)D);
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    double* acc = (double*)malloc(sizeof(double) * (size_t)Dv);
    int max_len = 0;
    for (int b = 0; b < s->batch; b++) max_len = seqlens[b] > max_len ? seqlens[b] : max_len;
    double* score = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    int local_status = (kv && qrow && acc && score) ? ORACLE_OK : ORACLE_NOMEM;

#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
      if (local_status != ORACLE_OK) continue;
      const int64_t row = rows ? rows[r] : r;
      if (row < 0 || row >= total_rows) { local_status = ORACLE_BAD_ARG; continue; }
      const int i = (int)((row / s->num_heads) % s->seqlen_q);
      const int b = (int)(row / ((int64_t)s->num_heads * s->seqlen_q));
      const int L = seqlens[b];
      const int n = visible_keys(s, L, i);
      int lo = t_begin ? t_begin[b] : 0;
      int hi = t_end ? t_end[b] : L;
      if (lo < 0) lo = 0;
      if (hi > n) hi = n;

      for (int d = 0; d < D; d++) qrow[d] = q_value(s, q, (size_t)row * D + d);
      const double sigma = (double)s->softmax_scale;

      /* scaled logits and their maximum */
      double m = -INFINITY;
      for (int t = lo; t < hi; t++) {
        int st = gather_token(s, cache, kv_scale, block_table, b, t, kv);
        if (st != ORACLE_OK) { local_status = st; break; }
        double dot = 0.0;
        for (int d = 0; d < D; d++) dot += qrow[d] * kv[d];
        score[t] = sigma * dot;
        if (score[t] > m) m = score[t];
      }
      if (local_status != ORACLE_OK) continue;

      double* o = out + (size_t)r * Dv;
      if (hi <= lo) { /* empty window */
        for (int d = 0; d < Dv; d++) o[d] = 0.0;
        lse[r] = -INFINITY;
        continue;
      }
      /* log-sum-exp of the scaled logits */
      double z = 0.0;
      for (int t = lo; t < hi; t++) z += exp(score[t] - m);
      const double row_lse = m + log(z);
      lse[r] = row_lse;

      /* softmax-weighted sum of the latents */
      for (int d = 0; d < Dv; d++) acc[d] = 0.0;
      for (int t = lo; t < hi; t++) {
        gather_token(s, cache, kv_scale, block_table, b, t, kv);
        const double p = exp(score[t] - row_lse);
        for (int d = 0; d < Dv; d++) acc[d] += p * kv[d];
      }
      for (int d = 0; d < Dv; d++) o[d] = acc[d];
    }
#pragma omp critical
    {
      if (local_status != ORACLE_OK && status == ORACLE_OK) status = local_status;
    }
    free(kv);
    free(qrow);
    free(acc);
    free(score);
  }
  return status;
}

/*
 * Merge of partial results over disjoint token windows by their log-sum-exp
 * (handbook page: chunk results merged with LSE, as in context parallelism).
 * For each row: M = max_j lse_j, lse = M + ln sum_j exp(lse_j - M),
 * out = sum_j exp(lse_j - lse) * out_j.  Parts with lse_j = -inf carry no
 * weight; a row whose parts are all empty stays empty (lse = -inf, out = 0).
 *
 * out_parts: [nparts][nrows][dv]; lse_parts: [nparts][nrows]
 */
int oracle_lse_merge(int32_t nparts, int64_t nrows, int32_t dv, const double* out_parts, const double* lse_parts,
                     double* out, double* lse) {
  if (nparts < 1 || nrows < 0 || dv < 1 || !out_parts || !lse_parts || !out || !lse) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < nrows; r++) {
    double M = -INFINITY;
    for (int j = 0; j < nparts; j++) {
      const double l = lse_parts[(size_t)j * nrows + r];
      if (l > M) M = l;
    }
    double* o = out + (size_t)r * dv;
    for (int d = 0; d < dv; d++) o[d] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double z = 0.0;
    for (int j = 0; j < nparts; j++) z += exp(lse_parts[(size_t)j * nrows + r] - M);
    const double total = M + log(z);
    lse[r] = total;
    for (int j = 0; j < nparts; j++) {
      const double l = lse_parts[(size_t)j * nrows + r];
      if (l == -INFINITY) continue;
      const double w = exp(l - total);
      const double* oj = out_parts + ((size_t)j * nrows + r) * dv;
      for (int d = 0; d < dv; d++) o[d] += w * oj[d];
    }
  }
  return ORACLE_OK;
}
