/*
 * tq_sq.h — C ABI of the SpectralQuant (SQ) codec in libtq.so: a calibrated per-head eigenbasis
 * with per-dimension Gaussian Lloyd-Max codebooks, beside the TurboQuant codec of tq.h.
 *
 * What is computed ("Ablation, Statistical Inference, and Validation for KV-Cache Compression",
 * arXiv 2607.09683):
 *   §2 "SpectralQuant": from calibration tokens X (n_cal x d) of one head, C = XᵀX/n_cal; its
 *   eigenvectors U (eigenvalues λ descending) give z = Uᵀx; the first d_eff dimensions are the
 *   semantic ones, d_eff = round(tr(C)²/‖C‖_F²); water-filling minimises Σ λ_k 4^(-b_k) subject to
 *   Σ b_k = B (B = b·d_eff, §6) and b_k >= b_tail; the other d - d_eff dimensions take b_tail bits;
 *   K and V have separate bases; the score of a query is <Uᵀq, ẑ>.
 *   §7 "Spectral gap criterion": d_eff is trimmed at the first k with λ_{k-1}/λ_k > γ and capped.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - U is the full eigenbasis (the tail is the remaining eigenvectors); each eigenvector is signed
 *     so that its entry of largest magnitude is positive.
 *   - σ_k² = λ_k (floored at 1e-12·λ_1) and dimension k is quantised with the b_k-bit Lloyd-Max
 *     codebook of a unit Gaussian applied to u_k = z_k/σ_k: idx_k = #{thresholds <= u_k}.
 *   - Water-filling is greedy one bit at a time to the largest λ_k 4^(-b_k) below 8 bits, ties to the
 *     fewer bits, then the lower k.  round() is round-half-up.  d_eff >= 1.
 *   - A record is the fields idx_0 .. idx_{d-1} in basis order, LSB first at bit offsets Σ_{j<k} b_j,
 *     then (with a sketch) the m sketch bits and the fp16 norm, padded to 4·ceil((max over heads of
 *     Σ_k b_k + [m + 16]) / 32) bytes.  No vector norm is stored.
 *   - The model of stream st is head st % n_heads.
 *
 * Packed tensor: one caller-allocated device buffer of n_streams·n_tokens records [stream][token],
 * tq_sq_record_bytes() bytes each.  Errors, streams and alignment follow tq.h: all arguments are
 * checked before any HIP call, device pointers must be 16-byte aligned, launches are asynchronous,
 * and the library never allocates caller-visible memory.  A codec owns its device tables (built on
 * the device current at tq_sq_create) until tq_sq_destroy; it may be used from any thread.
 */
#ifndef TQ_SQ_H
#define TQ_SQ_H

#include "tq.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t d;         /* head_dim: 64 or 128 for the kernels; tq_sq_calibrate also takes 256 */
    int32_t n_heads;   /* one model per head */
    int32_t b;         /* nominal bits per semantic dimension, 1..8 */
    int32_t b_tail;    /* bits per tail dimension, 1..b */
    int32_t waterfill; /* 0: every semantic dimension gets b bits (uniform); 1: greedy water-filling */
    int32_t d_eff_max; /* cap on d_eff (the known rank); 0 = none */
    double gamma;      /* spectral-gap threshold; <= 0 disables the criterion (the pages use 10) */
    int32_t m;         /* rows of the selective QJL sketch on the semantic dimensions (SQU-QKV): 0 (none),
                          16, 32, 48 or 64; needs d_eff <= 32 in every head */
    uint64_t seed;     /* keys the ±1 sketch (SplitMix64 tag 4, as tq.h's generator) */
} tq_sq_params;

/* Calibrate one model per head on the host (no GPU call).
 *   x_cal   host fp32 [n_heads][n_cal][d], the calibration tokens of each head; n_cal >= 1
 *   basis   host fp64 [n_heads][d][d]: basis[h][j][k] = entry j of eigenvector k
 *   lambda  host fp64 [n_heads][d], eigenvalues descending
 *   bits    host int32 [n_heads][d], bits of each basis dimension
 *   d_eff   host int32 [n_heads]
 * Any output may be NULL.  TQ_EINVAL on a bad parameter or NULL x_cal. */
int tq_sq_calibrate(const tq_sq_params* p, const float* x_cal, int64_t n_cal, double* basis,
                    double* lambda, int32_t* bits, int32_t* d_eff);

typedef struct tq_sq_codec tq_sq_codec;

/* Build a codec's device tables on the current device from a model (normally the output of
 * tq_sq_calibrate; host arrays in the same layout; p->b, b_tail, waterfill, gamma and d_eff_max are
 * not used here).  With p->m > 0 the records also carry the selective QJL sketch ("Ablation,
 * Statistical Inference, and Validation for KV-Cache Compression", §2 "SpectralQuant", SQU-QKV): for
 * the residual e_z = z - ẑ on the first d_eff[h] dimensions, the m sign bits σ of S e_z with
 * S[i][k] = -1 iff bit 63 of word i·d + k of the (p->seed, tag 4, head) SplitMix64 stream, then
 * ||e_z|| rounded to fp16; the scores and the attention add sqrt(pi/2)/m · ||e_z|| · <S q_Z, 2σ - 1>
 * (q_Z the query's first d_eff coordinates in the basis).  d_eff ([n_heads]) may be NULL when
 * p->m = 0.  TQ_EUNSUPPORTED for a sketch with some d_eff[h] > 32.  TQ_EINVAL for d not in {64, 128},
 * bits outside 1..8, m not in {0, 16, 32, 48, 64}, d_eff[h] outside 1..d, a non-finite basis entry
 * or lambda, or a NULL pointer (eigenvalues below 1e-12·λ_1, rounding-level negatives included, are
 * floored there); TQ_EHIP if the upload fails.  *out is set only on success.  The encode, decode
 * and scores calls return TQ_EINVAL unless that device is current. */
int tq_sq_create(const tq_sq_params* p, const double* basis, const double* lambda, const int32_t* bits,
                 const int32_t* d_eff, tq_sq_codec** out);

/* Free the codec's device tables.  No work using it may be pending.  NULL is a no-op. */
void tq_sq_destroy(tq_sq_codec* codec);

/* Bytes of one packed record (host only). */
int tq_sq_record_bytes(const tq_sq_codec* codec, int64_t* bytes);

/* Encode x [n_streams][n_tokens][d] (BF16; TQ_EUNSUPPORTED for other dtypes) into `packed`
 * [n_streams][n_tokens] records: z = Uᵀx on fp16 MFMA (x exact after a per-vector power-of-two
 * scale, U as an fp16 hi + lo pair, fp32 accumulation), then each dimension's codebook search and
 * the variable-width packing. */
int tq_sq_encode(const tq_sq_codec* codec, const void* x, tq_dtype x_dtype, int64_t n_streams,
                 int64_t n_tokens, void* packed, void* stream);

/* Decode x̂ = U ẑ, ẑ_k = σ_k c_{b_k}[idx_k], into x_hat [n_streams][n_tokens][d] (F32 or BF16). */
int tq_sq_decode(const tq_sq_codec* codec, const void* packed, int64_t n_streams, int64_t n_tokens,
                 void* x_hat, tq_dtype out_dtype, void* stream);

/* Workspace for tq_sq_qk_scores (the queries projected onto the basis). */
size_t tq_sq_scores_workspace_bytes(const tq_sq_codec* codec, int64_t n_streams, int64_t n_q);

/* Unscaled score estimates scores[st][i][t] = <Uᵀq[st][i], ẑ_t> = <q, x̂_t> on the packed keys.
 * q: [n_streams][n_q][d] F32 or BF16, n_q <= 256; scores: fp32 [n_streams][n_q][n_tokens].
 * The products run on fp16 MFMA with fp32 accumulation (relative error ~1e-3 or better). */
int tq_sq_qk_scores(const tq_sq_codec* codec, const void* q, tq_dtype q_dtype, int64_t n_q,
                    const void* packed_k, int64_t n_streams, int64_t n_tokens, float* scores,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for tq_sq_decode_attention (projected queries and split-K partials); a function of
 * the arguments only. */
size_t tq_sq_attention_workspace_bytes(const tq_sq_codec* ck, int32_t batch, int32_t n_q_heads,
                                       int32_t n_kv_heads, int64_t n_tokens);

/* One decode step of GQA attention over SpectralQuant caches ("Ablation...", §2 eq. (1) with the
 * SpectralQuant score <U_Kᵀq, ẑ_K> and values x̂_V = U_V ẑ_V):
 *   out[b][h] = Σ_t softmax_t(<U_Kᵀq[b][h], ẑ_K,t> · scale) · x̂_V,t,   scale = softmax_scale or 1/sqrt(d)
 * kv head = h / (n_q_heads/n_kv_heads); stream = b·n_kv_heads + kv head for both packed tensors (laid
 * out for n_tokens per stream); the weights are applied to ẑ_V in the V basis and U_V is applied once
 * per output row.  lengths: NULL, or a device pointer to `batch` int32 values (4-byte aligned)
 * clamped to [0, n_tokens]: element b attends to its first lengths[b] tokens, and a length of 0 gives
 * zero outputs.  q: [batch][n_q_heads][d] F32 or BF16; out: same shape, F32 or BF16.  ck and cv must
 * have n_heads == n_kv_heads and equal d; n_q_heads / n_kv_heads <= 16.  Products on fp16 MFMA with
 * fp32 accumulation (relative error ~1e-3). */
int tq_sq_decode_attention(const tq_sq_codec* ck, const tq_sq_codec* cv, const void* q, tq_dtype q_dtype,
                           int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                           const void* packed_v, int64_t n_tokens, const int32_t* lengths,
                           float softmax_scale, void* out, tq_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Host copies of the b-bit Lloyd-Max codebook of a unit Gaussian the kernels use (no GPU call):
 * thresholds[2^b - 1] and centroids[2^b] ascending, fp64; either may be NULL.  TQ_EINVAL unless
 * 1 <= b <= 8. */
int tq_sq_host_codebook(int32_t b, double* thresholds, double* centroids);

#ifdef __cplusplus
}
#endif

#endif /* TQ_SQ_H */
