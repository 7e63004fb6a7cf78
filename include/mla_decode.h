/*
 * mla_decode.h -- C ABI of libmla_decode.so: multi-head latent attention (MLA)
 * decode on the absorb path for AMD Instinct MI355X (gfx950).
 *
 * The operation.  Every cached token holds 576 numbers: a 512-wide latent c
 * followed by a 64-wide RoPE key k^R shared by all heads.  Each query row holds
 * the absorbed query q~ = [W_UK^T q^N ; q^R] (576 numbers, latent part first).
 * For a query row and the cached tokens t it may see,
 *     s_t = softmax_scale * (q~ . [c_t ; k^R_t]),
 *     out = sum_t softmax(s)_t * c_t          (512 numbers, in latent space),
 *     lse = ln sum_t exp(s_t).
 * ("MLA inference: two computation paths and FlashMLA": section "Two
 * equivalent paths", score equation and path two -- 128 query heads share one
 * 576-wide key and one 512-wide value; FlashMLA paragraph -- paged KV with
 * 64-token blocks, metadata computed from the context lengths, split-KV with a
 * merge of the partial results.  "FlashMLA: Fast Hopper Decoding for Latent
 * Attention Guide": Architecture, steps 1-4 -- the paged 512 + 64 cache read
 * straight from HBM, the two score parts summed and scaled by 1/sqrt(192),
 * online softmax, per-request sequence lengths.)  W_UK and W_UV themselves are
 * applied outside this library: it consumes q~ and produces the latent output.
 *
 * Three calls make one decode step:
 *   1. mla_get_workspace  -- size query (host only), then the split plan (device);
 *   2. mla_decode_fwd     -- the attention kernel over the paged cache;
 *   3. mla_splitkv_combine -- LSE merge of requests that the plan split.
 * The plan depends only on the sequence lengths and the parameters, so one plan
 * serves every layer of a step.
 *
 * Conventions for every call:
 *  - All pointers except `p` and `workspace_bytes` are device pointers, owned by
 *    the caller.  The library never allocates device memory and keeps no mutable
 *    global state.  Inputs are never written.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream).  Results are valid once that stream has reached the point
 *    after the last call.
 *  - The return value is an mla_status, decided synchronously.  Argument and
 *    shape errors return before anything is enqueued.  A failed launch returns
 *    MLA_ERR_HIP.  Nothing is thrown and nothing aborts.
 *  - Device-side values are not validated synchronously (that would need a host
 *    sync).  The kernels never read outside the buffers the parameters describe:
 *    sequence lengths are clamped to [0, max_blocks_per_seq * page_size], and a
 *    block-table entry outside [0, num_pages) is not dereferenced, and a plan
 *    is used only if its header matches the call's parameters.  Each event
 *    sets a bit in the workspace that mla_workspace_flags() reports.
 *  - Calls on distinct workspaces may run concurrently; calls sharing a
 *    workspace must be ordered on one stream.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,          /* null pointer, negative or inconsistent size */
  MLA_ERR_UNSUPPORTED = -2,          /* valid, but outside what the kernels implement */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3,  /* workspace_bytes below the size query's answer */
  MLA_ERR_HIP = -4,                  /* a HIP runtime call or kernel launch failed */
  MLA_ERR_SCRATCH_TOO_SMALL = -5     /* mla_decode_noalloc: the step needs more than its fixed scratch */
} mla_status;

/* Cache element type ("MLA inference ...": FlashMLA paragraph and exercise 2 --
 * FP8 KV support; "MLA and FP8 MoE Serving": E4M3 has 1 sign, 4 exponent and 3
 * mantissa bits and a largest value of 448). */
typedef enum {
  MLA_KV_BF16 = 0,        /* cache holds bf16 values */
  MLA_KV_FP8_E4M3FN = 1   /* cache holds OCP E4M3FN codes; value = decode(code) * kv_scale[page][slot] */
} mla_kv_dtype;

/* How an FP8 cache is multiplied (no effect on a bf16 cache). */
typedef enum {
  MLA_FP8_PATH_EXACT = 0,  /* codes widened to bf16 exactly, bf16 MFMAs, scale applied in fp32: the bf16
                              path's rounding only (one bf16 rounding of each softmax weight) */
  MLA_FP8_PATH_MFMA = 1    /* both products on E4M3 MFMAs ("MLA inference ...": Exercises, answer 2 -- FP8
                              tensor cores for the absorbed decode, with careful handling of precision):
                              q~ kept as a per-row scale times a sum of two E4M3 numbers (about 2^-8 of
                              q~), and each softmax weight times its token's scale times a power of two
                              rounded once to E4M3 (3 mantissa bits) for the value product; the running
                              maximum is raised whenever a score passes it by a factor 8, so the weights
                              that matter stay in E4M3's normal range.  Relative L2 error of the output about 1.5e-2 on
                              random inputs, against the oracle's exact result */
} mla_fp8_path;

/* Bits reported by mla_workspace_flags(). */
#define MLA_FLAG_SEQLEN_CLAMPED 0x1  /* some seqlens[b] was < seqlen_q or > max_blocks_per_seq * page_size */
#define MLA_FLAG_BAD_BLOCK      0x2  /* some referenced block-table entry was outside [0, num_pages) */
#define MLA_FLAG_BAD_PLAN       0x4  /* the workspace holds no plan, or one made for other parameters (batch,
                                        seqlen_q * num_heads, workgroup count or max_blocks_per_seq): the decode
                                        wrote out = 0 and lse = -inf for every row and read nothing else */

typedef struct {
  int32_t batch;               /* B >= 1: requests in the step */
  int32_t seqlen_q;            /* s_q in [1, 8]: new tokens per request */
  int32_t num_heads;           /* H in [1, 128]: query heads; rows per request = s_q * H */
  int32_t head_dim_qk;         /* must be 576 (512 latent + 64 RoPE) */
  int32_t head_dim_v;          /* must be 512 (the latent part of each cache row) */
  int32_t page_size;           /* must be 64 tokens */
  int32_t num_pages;           /* P >= 1: physical pages in kv_cache */
  int32_t max_blocks_per_seq;  /* >= 1: row stride of block_table */
  int32_t kv_dtype;            /* an mla_kv_dtype */
  int32_t causal;              /* nonzero: new token i of a request sees L - s_q + 1 + i keys; else all L */
  float softmax_scale;         /* > 0, e.g. 1/sqrt(192) */
  int32_t num_workgroups;      /* 0: one persistent workgroup per compute unit (the default);
                                  > 0: use that many (tests use it to force other split plans) */
  int32_t fp8_path;            /* an mla_fp8_path; must be MLA_FP8_PATH_EXACT for a bf16 cache */
} mla_decode_params;

/*
 * Split plan.  The pages of all requests are laid end to end and cut into one
 * contiguous stretch per persistent workgroup, balanced on pages plus a fixed
 * cost per request (the FlashMLA paragraph's scheduling metadata: which stretch
 * of KV each compute unit handles, decided from the context lengths).  A request
 * cut by a stretch boundary is computed in pieces and merged by
 * mla_splitkv_combine.
 *
 * workspace == NULL: writes the required size in bytes to *workspace_bytes and
 *   returns; no device work.  The size depends on p only (and on the device's
 *   compute-unit count when p->num_workgroups == 0).
 * workspace != NULL: *workspace_bytes must hold at least that size.  Enqueues
 *   the plan kernel on `stream`; it reads seqlens (device int32 [batch]: tokens
 *   per request, counting the s_q new ones) and writes the plan into workspace.
 *   workspace must be 256-byte aligned.
 */
int mla_get_workspace(const mla_decode_params* p, const int32_t* seqlens, void* workspace,
                      size_t* workspace_bytes, void* stream);

/*
 * The attention kernel.  Requires a plan made by mla_get_workspace with the same
 * p and the same seqlens contents, earlier on the same stream.
 *
 * q:           bf16 [batch][seqlen_q][num_heads][576], the absorbed queries
 * kv_cache:    [num_pages][64][576] of bf16 (MLA_KV_BF16) or E4M3FN bytes (MLA_KV_FP8_E4M3FN);
 *              token t of request b is row t % 64 of page block_table[b][t / 64]
 * kv_scale:    fp32 [num_pages][64], per-token scale of an FP8 cache, 16-byte aligned; must be NULL for bf16.
 *              The kernel widens each code to bf16 exactly and applies the scale in fp32 to the
 *              token's score and to its softmax weight before that weight is rounded to bf16.
 * block_table: int32 [batch][max_blocks_per_seq]; entries past the last page of a request are not read
 * seqlens:     int32 [batch], the same buffer contents the plan read
 * out:         bf16 [batch][seqlen_q][num_heads][512]
 * Alignment: q, kv_cache and kv_scale 16 bytes, out 8 bytes, workspace 256 bytes
 * (MLA_ERR_INVALID_ARG otherwise).
 * lse:         fp32 [batch][seqlen_q][num_heads], natural log of the softmax normaliser of the scaled scores
 * Rows of requests the plan did not split are final after this call; the others
 * are final after mla_splitkv_combine.
 */
int mla_decode_fwd(const mla_decode_params* p, const void* q, const void* kv_cache, const float* kv_scale,
                   const int32_t* block_table, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                   void* out, float* lse, void* stream);

/*
 * LSE merge of split requests ("MLA inference ...": the chunked-prefix and
 * split-KV passages -- partial results over disjoint stretches of KV merged by
 * their LSE).  For each row of a split request:
 *   M = max_j lse_j,  lse = M + ln sum_j exp(lse_j - M),  out = sum_j exp(lse_j - lse) * out_j.
 * Writes out and lse (same layouts as above) for split requests only; other rows
 * are left as mla_decode_fwd wrote them.  After this call every element of out
 * and lse has been written.
 */
int mla_splitkv_combine(const mla_decode_params* p, const void* workspace, size_t workspace_bytes, void* out,
                        float* lse, void* stream);

/*
 * Synchronously reads the MLA_FLAG_* bits the last plan and decode set in
 * workspace (waits for `stream` first).  *flags receives the bits.
 */
int mla_workspace_flags(const void* workspace, uint32_t* flags, void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: one whole
 * decode step (the split plan, mla_decode_fwd and mla_splitkv_combine) with its
 * workspace in a fixed array of MLA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  Nothing is allocated:
 * no hipMalloc, no hipFree, no allocating library call.  The arguments are those
 * of mla_decode_fwd without the workspace; results are the same bits.
 *
 * Returns MLA_ERR_SCRATCH_TOO_SMALL, before anything is enqueued, when the
 * step's workspace (the size mla_get_workspace reports for p) exceeds the
 * array: with the default workgroup count that is about 65 MiB at any batch up
 * to 8192 and any s_q * num_heads, so only a large explicit num_workgroups is
 * rejected.  Every call on one GPU uses that GPU's one array, which keeps the
 * last call's plan and partial results: calls ordered on one stream are safe;
 * calls that overlap on one GPU (other streams, other threads) race.  The flag
 * bits of mla_workspace_flags are not reported for this path.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
int mla_decode_noalloc(const mla_decode_params* p, const void* q, const void* kv_cache, const float* kv_scale,
                       const int32_t* block_table, const int32_t* seqlens, void* out, float* lse, void* stream);

/* Static description of a status code. */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
