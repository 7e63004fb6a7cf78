/*
 * mla_prefill.h -- the expand path of MLA for one request's new tokens
 * (prefill or extend), in libmla_decode.so (gfx950).
 *
 * "MLA inference: two computation paths and FlashMLA", section "Two
 * equivalent paths", path one: the cached latents are expanded with W_UK and
 * W_UV into every head's keys and values and ordinary multi-head attention
 * runs with 192-wide queries/keys and 128-wide values.  The same page's
 * engine discussion (SGLang's chunked-prefix method) expands a long prefix in
 * chunks, attends chunk by chunk and merges the chunks with their LSEs, the
 * merge used for split-KV.
 *
 * One request per call.  Its L cached tokens (prefix and new tokens; the new
 * tokens' latents are already in the cache) sit in the paged cache of
 * mla_decode.h: bf16 [P][64][576], token t of the request at
 * cache[block_table[t / 64]][t % 64], latent c in numbers 0..511 and the shared
 * RoPE key k^R in 512..575.  Its n new tokens are the last n positions; new
 * token i (position L - n + i) attends to the keys at positions <= L - n + i.
 *
 *   expansion of token t, head h:   k[h][t] = [ W_UK[h] c_t ; k^R_t ]   (192)
 *                                   v[h][t] = W_UV[h] c_t               (128)
 *   attention of new token i, head h over the keys it sees:
 *       s_t = scale * q[i][h] . k[h][t],  out = sum_t softmax(s)_t v[h][t],
 *       lse = ln sum_t exp(s_t)
 *
 * Conventions as in mla_decode.h: caller-owned device pointers, nothing
 * allocated, work enqueued on `stream`, an mla_status returned synchronously
 * (argument errors before anything is enqueued); inputs are never written.
 * bf16 tensors are 16-byte aligned; products accumulate in fp32.
 */
#ifndef MLA_PREFILL_H
#define MLA_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t num_heads;     /* H in [1, 128] */
  int32_t num_new;       /* n in [1, 65536]: new tokens of the request (query rows per head) */
  int32_t seqlen;        /* L in [n, max_blocks * 64]: tokens of the request in the cache */
  int32_t num_pages;     /* P: pages in the cache (block-table entries are checked against it) */
  int32_t max_blocks;    /* entries in the request's block-table row */
  int32_t chunk_tokens;  /* Tc: tokens expanded per chunk, a multiple of 64 in [64, 65536] */
  float softmax_scale;   /* e.g. 1/sqrt(192) */
  int32_t d_nope;        /* must be 128 */
  int32_t d_rope;        /* must be 64 */
  int32_t d_latent;      /* must be 512 */
  int32_t d_v;           /* must be 128 */
} mla_prefill_params;

/*
 * Expand tokens [t0, t0 + ntok) of the request (0 <= t0, 1 <= ntok, t0 + ntok <= L).
 * kv_cache:    bf16 [P][64][576]; block_table: int32 [max_blocks] (the request's row)
 * w_uk, w_uv:  bf16 [H][128][512] (row n of W_UK[h] multiplies c into k^N[n])
 * k_out:       bf16 [H][ld][192], ld = ntok rounded up to a multiple of 64; token j of the
 *              range is row j; rows ntok..ld-1 are written as zeros
 * vt_out:      bf16 [H][128][ld]: v transposed (dims-major, tokens contiguous), zero-padded
 * Returns MLA_ERR_INVALID_ARG for null/misaligned pointers or a range outside [0, L),
 * MLA_ERR_UNSUPPORTED for other widths.  A block-table entry outside [0, P) is read as page 0
 * and reported in no flag: the caller validates its tables.
 */
int mla_expand_kv(const mla_prefill_params* p, const void* kv_cache, const int32_t* block_table, int32_t t0,
                  int32_t ntok, const void* w_uk, const void* w_uv, void* k_out, void* vt_out, void* stream);

/*
 * Attention of the n new tokens over the expanded keys of positions [t0, t0 + ntok).
 * q:    bf16 [n][H][192]  ([q^N ; q^R] per head)
 * k, vt: as written by mla_expand_kv for the same range
 * out:  fp32 [n][H][128]  normalised over the keys of this range that the row sees
 * lse:  fp32 [n][H]       natural-log LSE over those keys; a row that sees none gets
 *                          out = 0 and lse = -inf (it then carries no weight in a merge)
 */
int mla_prefill_attention(const mla_prefill_params* p, const void* q, const void* k, const void* vt, int32_t t0,
                          int32_t ntok, float* out, float* lse, void* stream);

/*
 * LSE merge of J partial results over disjoint key ranges (the split-KV merge):
 *   M = max_j lse_j, lse = M + ln sum_j exp(lse_j - M), out = sum_j exp(lse_j - lse) out_j.
 * out_parts: fp32 [J][rows][128]; lse_parts: fp32 [J][rows]; out: bf16 [rows][128];
 * lse: fp32 [rows].  Parts with lse = -inf carry no weight; a row with no part gets
 * out = 0, lse = -inf.  1 <= J <= 4096, 1 <= rows <= 2^24.
 */
int mla_lse_merge(int32_t rows, int32_t nparts, const float* out_parts, const float* lse_parts, void* out,
                  float* lse, void* stream);

/* Workspace bytes mla_chunked_prefill needs for these parameters (one K and one V chunk,
 * the fp32 partials and LSEs of every chunk). */
int mla_prefill_workspace_size(const mla_prefill_params* p, size_t* bytes);

/*
 * The whole expand path, chunk by chunk: for each chunk of chunk_tokens positions,
 * mla_expand_kv then mla_prefill_attention into the chunk's partial, then one
 * mla_lse_merge.  When one chunk covers the whole context (chunk_tokens >= seqlen)
 * the attention writes out and lse itself and no merge runs (the same numbers: a
 * merge of a single part only rounds it to bf16).  q: bf16 [n][H][192]; out: bf16
 * [n][H][128]; lse: fp32 [n][H].
 * workspace: device memory of at least mla_prefill_workspace_size bytes, 256-byte aligned.
 */
int mla_chunked_prefill(const mla_prefill_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                        const void* w_uk, const void* w_uv, void* workspace, size_t workspace_bytes, void* out,
                        float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PREFILL_H */
