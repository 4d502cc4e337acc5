/*
 * tq_fmag.h — C ABI of the Fourier-magnitude codec (Fmag) in libtq.so, beside the TurboQuant codec of
 * tq.h and the SpectralQuant codec of tq_sq.h.
 *
 * What is computed ("Fourier Magnitude KV Cache Quantization", forum thread, "Method" of its first
 * post): each vector's FFT along head_dim; its magnitude spectrum quantised to b bits by min-max; the
 * phase kept at bf16 or quantised to p bits ("Fmag4+phase8b", "phase6b"); reconstruction by the
 * inverse FFT of mag_q·(cos φ + i sin φ).
 *
 * Conventions fixed by this library where the thread is silent:
 *   - The real FFT X_k = Σ_j x_j e^{-2πi jk/d}, k = 0..d/2, inverted by the real inverse FFT.
 *   - Min-max per vector over the d/2 + 1 magnitudes: q_k = floor((|X_k| - lo)/(hi - lo)·(2^b - 1)
 *     + 1/2) (0 when hi = lo); lo and hi stored as fp32.
 *   - A p-bit phase is the nearest of the angles -π + 2π i/2^p (index mod 2^p); p = 16 stores the
 *     phase rounded to bf16.
 *   - Record: the d/2 + 1 magnitude fields (b bits), then the d/2 + 1 phase fields (p bits), LSB first,
 *     padded to a 32-bit word, then lo and hi: tq_fmag_record_bytes() bytes per vector, records
 *     [stream][token] in one caller buffer.
 *   - Scores are <q, x̂> computed in the frequency domain (Parseval): Σ_k w_k (Re Q_k Re X̂_k +
 *     Im Q_k Im X̂_k)/d with w = 1 at k = 0 and d/2, else 2.
 *
 * Errors, streams and alignment follow tq.h: all arguments are checked before any HIP call, device
 * pointers are 16-byte aligned, launches are asynchronous on `stream`, the library never allocates
 * caller-visible memory; its read-only tables are cached per (device, d, b, p) and freed by
 * tq_clear_cache().
 */
#ifndef TQ_FMAG_H
#define TQ_FMAG_H

#include "tq.h"

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_FMAG_PHASE_BF16 16

typedef struct {
    int32_t d; /* head_dim: 64 or 128 */
    int32_t b; /* magnitude bits, 1..8 */
    int32_t p; /* phase bits, 1..8, or TQ_FMAG_PHASE_BF16 */
} tq_fmag_params;

/* Bytes of one record (host only). */
int tq_fmag_record_bytes(const tq_fmag_params* p, int64_t* bytes);

/* Encode x [n_streams][n_tokens][d] (BF16; TQ_EUNSUPPORTED otherwise) into `packed`. The DFT runs on
 * fp16 MFMA (x exact after a per-vector power-of-two scale, the DFT matrix as an fp16 hi + lo pair,
 * fp32 accumulation); magnitudes, phases (an fp32 atan2 within 5e-7 rad) and the min-max in fp32. */
int tq_fmag_encode(const tq_fmag_params* p, const void* x, tq_dtype x_dtype, int64_t n_streams,
                   int64_t n_tokens, void* packed, void* stream);

/* Decode x̂ = irfft(mag_q·e^{iφ_q}) into x_hat [n_streams][n_tokens][d] (F32 or BF16); the inverse
 * DFT runs on fp16 MFMA with hi + lo operands (about 2^-21 relative). */
int tq_fmag_decode(const tq_fmag_params* p, const void* packed, int64_t n_streams, int64_t n_tokens,
                   void* x_hat, tq_dtype out_dtype, void* stream);

/* Workspace for tq_fmag_qk_scores (the queries' weighted spectra). */
size_t tq_fmag_scores_workspace_bytes(const tq_fmag_params* p, int64_t n_streams, int64_t n_q);

/* scores[st][i][t] = <q[st][i], x̂_t>; q: [n_streams][n_q][d] F32 or BF16, n_q <= 256; fp16 MFMA
 * products with fp32 accumulation (relative error ~1e-3). */
int tq_fmag_qk_scores(const tq_fmag_params* p, const void* q, tq_dtype q_dtype, int64_t n_q,
                      const void* packed, int64_t n_streams, int64_t n_tokens, float* scores,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for tq_fmag_decode_attention (projected queries and per-split partials). */
size_t tq_fmag_attention_workspace_bytes(const tq_fmag_params* pk, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t n_tokens);

/* Decode-step attention over Fmag K and V caches ("Method": attention runs on the reconstructed
 * cache): out[b][h] = Σ_t softmax_t(scale·<q[b][h], x̂_K,t>)·x̂_V,t over the first lengths[b] tokens
 * (all n_tokens when lengths is NULL; a row with no token is 0).  K and V may use different b and p,
 * with the same d.  q: [batch][n_q_heads][d] F32 or BF16; packed_k / packed_v: [batch·n_kv_heads]
 * streams of n_tokens records; query head h reads kv head h / (n_q_heads / n_kv_heads), at most 16
 * query heads per kv head; softmax_scale 0 means 1/sqrt(d); out [batch][n_q_heads][d] F32 or BF16.
 * The scores use the Parseval form of tq_fmag_qk_scores; the weighted sum is taken over the
 * reconstructed spectra (the inverse FFT is linear) and one inverse DFT per output row finishes it.
 * fp16 MFMA products with fp32 accumulation: relative error ~1e-3. */
int tq_fmag_decode_attention(const tq_fmag_params* pk, const tq_fmag_params* pv, const void* q, tq_dtype q_dtype,
                             int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                             const void* packed_v, int64_t n_tokens, const int32_t* lengths, float softmax_scale,
                             void* out, tq_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_FMAG_H */
