/*
 * mla_proj.h -- the two per-head projections on either side of the absorbed
 * attention core, in libmla_decode.so (gfx950).
 *
 * The absorb path ("MLA inference: two computation paths and FlashMLA",
 * section "Two equivalent paths", path two) folds W_UK into the query and
 * applies W_UV after the attention, in latent space.  For query row t (a
 * request's new token) and head h, with k^N = W_UK[h] c and v = W_UV[h] c for a
 * cached latent c (so W_UK[h] and W_UV[h] are 128 x 512):
 *     q~[t,h]  = [ W_UK[h]^T q^N[t,h] ; q^R[t,h] ]    (512 + 64 numbers, the
 *                                                      query mla_decode_fwd reads)
 *     out[t,h] = W_UV[h] o[t,h]                       (128 numbers, from the
 *                                                      512-wide latent output o)
 * Both are batched products with one small matrix per head (128 heads, M = the
 * query rows, K and N of 128 and 512); each reads its 16.8 MB of weights once,
 * so both are bound by HBM bandwidth on the weights.
 *
 * Conventions as in mla_decode.h: device pointers owned by the caller, nothing
 * allocated, work enqueued on `stream`, an mla_status returned synchronously
 * (argument errors before anything is enqueued).  Inputs are never written.
 * Every tensor is bf16, dense, in the layout given, 16-byte aligned.  The
 * products accumulate in fp32 and round once to bf16 (round to nearest even).
 */
#ifndef MLA_PROJ_H
#define MLA_PROJ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t tokens;      /* T in [1, 65536]: query rows per head (batch * s_q) */
  int32_t num_heads;   /* H in [1, 128] */
  int32_t d_nope;      /* must be 128: width of q^N and of a row of W_UK[h] */
  int32_t d_rope;      /* must be 64: width of q^R */
  int32_t d_latent;    /* must be 512: width of the latent (columns of W_UK[h] and W_UV[h]) */
  int32_t d_v;         /* must be 128: width of a head's output (rows of W_UV[h]) */
} mla_proj_params;

/*
 * Absorbed query.
 * q_nope:  bf16 [T][H][128]   q^N
 * q_rope:  bf16 [T][H][64]    q^R (copied into the last 64 numbers of each row)
 * w_uk:    bf16 [H][128][512] W_UK, row n of head h = W_UK[h][n][:]
 * q_tilde: bf16 [T][H][576]   out: [W_UK[h]^T q^N ; q^R], the q of mla_decode_fwd
 * Returns MLA_ERR_INVALID_ARG for a null or misaligned pointer or a size out of
 * range, MLA_ERR_UNSUPPORTED for other widths.
 */
int mla_absorb_q(const mla_proj_params* p, const void* q_nope, const void* q_rope, const void* w_uk, void* q_tilde,
                 void* stream);

/*
 * Output projection.
 * o_latent: bf16 [T][H][512]   the latent output of mla_decode_fwd / mla_splitkv_combine
 * w_uv:     bf16 [H][128][512] W_UV, row v of head h = W_UV[h][v][:]
 * out:      bf16 [T][H][128]   out: W_UV[h] o[t,h]
 * Errors as for mla_absorb_q.
 */
int mla_project_out(const mla_proj_params* p, const void* o_latent, const void* w_uv, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROJ_H */
