/*
 * tq.h — C ABI of the MI355X (gfx950) TurboQuant-family KV-cache codec, libtq.so.
 *
 * What is computed (sources cited by page title and section):
 *   "Ablation, Statistical Inference, and Validation for KV-Cache Compression" (arXiv 2607.09683),
 *   §2 Background, "TurboQuant" paragraph: each key/value vector k is sign-flipped with per-head
 *   random signs s, rotated y = WHT(k ⊙ s)/sqrt(d), and its coordinates (≈ Beta((d-1)/2,(d-1)/2)
 *   for a unit vector) are quantised with one analytical Lloyd-Max codebook shared by all
 *   coordinates; the WHT-domain residual e = y - ŷ can carry a 1-bit QJL sketch on the key path.
 *   §2 eq. (1): attention T = softmax(Q K^T / sqrt(d)) V.  §2 "SpectralQuant" paragraph: the
 *   asymmetric score estimator <q, k̂> + sqrt(pi/2)/m ||e|| q^T S sign(S e) (used here in the WHT
 *   domain with a Gaussian S).  §3.2 "Storage complexity": b·d bits per token.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - WHT = unnormalised Sylvester Hadamard matrix H in natural order; inverse s ⊙ (H ŷ)/sqrt(d).
 *   - Vectors are normalised by their exact norm n before rotation; n is stored as fp16 (RNE).
 *   - idx_j = #{i : t_i <= y_j} over the 2^b - 1 thresholds (ties go up), centroids ascending.
 *   - QJL (m > 0): z = S_h e with S_h an m x d matrix of N(0,1) draws rounded to fp16, or, with
 *     sketch = TQ_SKETCH_RHT, the randomized Hadamard sketch S_h = H diag(s2_h) (m = d; the pages'
 *     sign(WHT(e ⊙ s2))); e is the residual itself, taken into the projection as two fp16 parts
 *     (exact to ~2^-22 relative), so z is fp32-accurate: a bit can differ from the sign of the
 *     exact projection only where |z_i| < 1e-6.  Sketch bit i = [z_i >= 0] (sign(0) = +1); the fp16
 *     (RNE) norm ||e|| is stored too.  Scores and attention use the same estimator for both kinds.
 *   - Random tables: SplitMix64 (Steele, Lea, Flood 2014) keyed by (seed, tag, head); signs use
 *     tag 1 (s_j = -1 iff bit 63 of word j), S uses tag 2 with Box-Muller (1958) on word pairs, the
 *     RHT signs s2 use tag 3 like tag 1.
 *     The RNG head of stream st is st % n_heads.
 *
 * Packed tensor (one caller-allocated byte buffer, see tq_get_layout): four planes, each starting
 * on a 256-byte boundary, each indexed [stream][token]:
 *   idx    d·b/8 bytes per vector, a little-endian bit string with coordinate j at bits [j·b,(j+1)·b)
 *   sketch m/8 bytes per vector, bit i = sigma_i (LSB first); absent when m = 0
 *   norm   fp16 n per vector
 *   rnorm  fp16 ||e|| per vector; absent when m = 0
 *
 * Errors: every entry point validates all arguments before touching the GPU and returns TQ_OK (0)
 * or a negative TQ_E* code; nothing is launched on error.  Kernel launches are asynchronous on
 * `stream` (a hipStream_t; NULL = the null stream); device faults surface at the caller's next
 * synchronisation.  All device pointers are caller-owned and must be 16-byte aligned; the library
 * never allocates or frees caller-visible memory.  Internally it keeps a mutex-guarded cache of
 * read-only device tables (codebook, signs, S, search grid) per (device, d, b, m, n_heads, seed, sketch),
 * built on the host in fp64 on first use; tq_clear_cache() frees them.  Calls are thread-safe.
 * NaN/Inf inputs propagate unchecked.  A vector norm above 65504 is outside the fp16 norm format
 * and is stored as +Inf.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_OK 0
#define TQ_EINVAL (-1)       /* bad value: d not in {64,128,256}, b not in 1..8, m % 32, sketch, null ptr, n <= 0 */
#define TQ_EUNSUPPORTED (-2) /* valid but not built, e.g. an attention (b_K, b_V) pair not compiled */
#define TQ_EALIGN (-3)       /* a device pointer is not 16-byte aligned */
#define TQ_EWORKSPACE (-4)   /* workspace smaller than the matching *_workspace_bytes() */
#define TQ_EHIP (-5)         /* a HIP runtime call or kernel launch failed */

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* Rotation before quantisation (tq_params.rotation). */
#define TQ_ROTATION_WHT 0    /* y = WHT(x ⊙ s)/(sqrt(d) ||x||): TurboQuant ("Ablation...", §2 TurboQuant) */
#define TQ_ROTATION_NONE 1   /* y = x/||x||, the Beta codebook applied without rotation: the pages' Plain-KV
                                ("Ablation...", §4, surviving schemes) */

/* Kind of the QJL sketch matrix S_h (tq_params.sketch). */
#define TQ_SKETCH_GAUSSIAN 0 /* m rows of i.i.d. N(0,1) draws rounded to fp16 (tag 2) */
#define TQ_SKETCH_RHT 1      /* randomized Hadamard: S_h = H diag(s2_h), s2_h the signs of tag 3, m = d
                                ("Ablation...", §2 TurboQuant: b = sign(WHT(e ⊙ s2))) */

typedef struct {
    int32_t d;        /* head_dim: 64, 128 or 256 */
    int32_t b;        /* codebook bits per coordinate, 1..8 */
    int32_t m;        /* QJL sketch rows; 0 = no sketch; a multiple of 32, at most d (= d for RHT) */
    int32_t n_heads;  /* heads with distinct random state; stream st uses head st % n_heads */
    uint64_t seed;    /* keys the random signs and S */
    int32_t sketch;   /* TQ_SKETCH_GAUSSIAN or TQ_SKETCH_RHT; ignored when m = 0 */
    int32_t rotation; /* TQ_ROTATION_WHT (0) or TQ_ROTATION_NONE; scores, attention and decode use the
                         same domain as the encode */
} tq_params;

typedef struct {
    int64_t idx_bytes_per_vec;     /* d·b/8 */
    int64_t sketch_bytes_per_vec;  /* m/8 */
    int64_t off_idx, off_sketch, off_norm, off_rnorm; /* byte offsets of the planes */
    int64_t total_bytes;           /* bytes the caller allocates for one packed tensor */
} tq_layout;

/* Packed-buffer geometry for n_streams x n_tokens vectors (host only, no GPU call). */
int tq_get_layout(const tq_params* p, int64_t n_streams, int64_t n_tokens, tq_layout* out);

/* Encode x [n_streams][n_new][d] (F32 or BF16) as tokens [t0, t0 + n_new) of every stream of a packed
 * tensor laid out for n_streams x capacity tokens (tq_get_layout with n_tokens = capacity); the other
 * tokens' records are left untouched, so a cache can grow one decode step (or one chunk) at a time.
 * TQ_EINVAL unless 0 <= t0 and t0 + n_new <= capacity.  Otherwise as tq_encode. */
int tq_encode_append(const tq_params* p, const void* x, tq_dtype x_dtype, int64_t n_streams,
                     int64_t n_new, void* packed, int64_t capacity, int64_t t0, void* stream);

/* Encode x [n_streams][n_tokens][d] (F32 or BF16) into `packed` (layout from tq_get_layout).
 * Steps per vector: norm, sign flip, WHT, scale, Lloyd-Max search, bit-pack, and with m > 0 the
 * residual, S·e and its sign bits ("Ablation...", §2 TurboQuant). */
int tq_encode(const tq_params* p, const void* x, tq_dtype x_dtype, int64_t n_streams,
              int64_t n_tokens, void* packed, void* stream);

/* Encode the keys k and the values v of the same tokens, both [n_streams][n_tokens][d] of x_dtype,
 * into packed_k (layout of pk) and packed_v (layout of pv): the same records, byte for byte, as
 * tq_encode(pk, k, ...) followed by tq_encode(pv, v, ...) ("Ablation...", §2 TurboQuant: every key
 * and value vector of the cache is encoded).  For bf16 input with the same d <= 128 and b <= 4 on
 * both sides, the Walsh-Hadamard rotation, no value sketch and a key sketch that fits the kernel's
 * tables (Gaussian with m <= 128, or randomized Hadamard), one launch encodes both: each wave takes
 * a group of keys and then the values of the same tokens, so the value stream's HBM traffic runs
 * while the key sketch holds the vector units.  Otherwise the two encodes run one after the other
 * on `stream`.  The caller owns every buffer.  Errors: those of tq_encode for either side, checked
 * before any launch. */
int tq_encode_kv(const tq_params* pk, const tq_params* pv, const void* k, const void* v,
                 tq_dtype x_dtype, int64_t n_streams, int64_t n_tokens, void* packed_k,
                 void* packed_v, void* stream);

/* tq_encode_kv into tokens [t0, t0 + n_new) of caches laid out for `capacity` tokens per stream
 * (layouts of pk and pv at n_streams x capacity): the same records as tq_encode_append on each
 * side, in one launch under the same conditions (the decode step's append of one key and one value
 * per stream is one launch).  TQ_EINVAL unless 0 <= t0 and t0 + n_new <= capacity; otherwise as
 * tq_encode_kv. */
int tq_encode_kv_append(const tq_params* pk, const tq_params* pv, const void* k, const void* v,
                        tq_dtype x_dtype, int64_t n_streams, int64_t n_new, void* packed_k,
                        void* packed_v, int64_t capacity, int64_t t0, void* stream);

/* Decode the MSE reconstruction x̂ = n16 · s ⊙ (H c[idx]) / sqrt(d) into x_hat
 * [n_streams][n_tokens][d] (F32 or BF16).  The QJL sketch is not applied. */
int tq_decode(const tq_params* p, const void* packed, int64_t n_streams, int64_t n_tokens,
              void* x_hat, tq_dtype out_dtype, void* stream);

/* Decode with the QJL correction added in the rotated domain ("Ablation...", §2 TurboQuant: the
 * sketch correction sqrt(pi/2)/d ||e|| s2 ⊙ WHT(b) is added at decode):
 *   x̂ = n16 · s ⊙ H (c[idx] + Δŷ) / sqrt(d),   Δŷ = sqrt(pi/2)/m · r16 · S^T (2σ - 1),
 * for either sketch kind (for the RHT sketch S^T (2σ - 1) = s2 ⊙ H (2σ - 1), m = d).  Same arguments,
 * layout and ownership as tq_decode; p->m must be > 0 (TQ_EINVAL otherwise).  S^T is held in LDS
 * (d·m·2 bytes, 128 KiB at d = m = 256); every supported (d, b, m) fits. */
int tq_decode_qjl(const tq_params* p, const void* packed, int64_t n_streams, int64_t n_tokens,
                  void* x_hat, tq_dtype out_dtype, void* stream);

/* Workspace for tq_qk_scores (rotated queries and their S-projections). */
size_t tq_scores_workspace_bytes(const tq_params* pk, int64_t n_streams, int64_t n_q);

/* Unscaled score estimates scores[st][i][t] ≈ <q[st][i], k[st][t]> on the packed keys:
 *   n16·(<q_rot, c[idx]> + sqrt(pi/2)/m · r16 · <S q_rot, 2σ-1>),  q_rot = H(q ⊙ s)/sqrt(d)
 * ("Ablation...", §2 TurboQuant and SpectralQuant paragraphs).  q: [n_streams][n_q][d] F32/BF16;
 * n_q <= 256.  Computed in fp32 from fp16 operands (relative error ~1e-3 or better). */
int tq_qk_scores(const tq_params* pk, const void* q, tq_dtype q_dtype, int64_t n_q,
                 const void* packed_k, int64_t n_streams, int64_t n_tokens, float* scores,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for tq_decode_attention (query operands and split-K partials). */
size_t tq_attention_workspace_bytes(const tq_params* pk, int32_t batch, int32_t n_q_heads,
                                    int32_t n_kv_heads, int64_t n_tokens);

/* One decode step of GQA attention over the compressed cache ("Ablation...", eq. (1)):
 *   out[b][h] = Σ_t softmax_t(ŝ(q[b][h], K_t) · scale) · x̂^V_t,   scale = softmax_scale or 1/sqrt(d)
 * with ŝ the score estimate above and x̂^V the decoded values; kv head = h / (n_q_heads/n_kv_heads);
 * stream = b·n_kv_heads + kv head for both packed tensors.  q: [batch][n_q_heads][d] BF16 or F32;
 * out: same shape, BF16 or F32.  pv->m must be 0; pk->d == pv->d; n_heads of both == n_kv_heads;
 * n_q_heads / n_kv_heads <= 16.  Values are accumulated in the rotated domain and rotated back once.
 * One stream's packed K index plane (n_tokens·d·b_K/8 bytes) and V index plane must stay below
 * 2^32 - 2^16 bytes (32-bit buffer offsets within a stream): TQ_EUNSUPPORTED beyond. */
int tq_decode_attention(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype,
                        int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                        const void* packed_k, const void* packed_v, int64_t n_tokens,
                        float softmax_scale, void* out, tq_dtype out_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* tq_decode_attention over caches of different lengths: batch element b attends to its first
 * lengths[b] tokens only (a decode step over sequences of different lengths).
 * lengths: device pointer to `batch` int32 values, 4-byte aligned, read by the kernels on `stream`;
 * values are clamped to [0, n_tokens] (the capacity the packed tensors are laid out for, which also
 * sizes the workspace); a length of 0 gives zero outputs for that batch element.  NULL = every
 * element has n_tokens tokens, as tq_decode_attention.  Everything else as tq_decode_attention. */
int tq_decode_attention_varlen(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype,
                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                               const void* packed_v, int64_t n_tokens, const int32_t* lengths,
                               float softmax_scale, void* out, tq_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Allocation-free tq_decode_attention_varlen, for callers that cannot allocate device memory (code
 * under HIP graph capture, allocation-free serving loops, harnesses that forbid hipMalloc).
 * Arguments, layouts, results and errors as tq_decode_attention_varlen, without the workspace: the
 * query operands and split partials live in a device array inside the library, one per GPU, of
 * tq_attention_noalloc_max_bytes() bytes (32 MiB, held from the first call on a device until the
 * process ends; the decode step of batch 16 x 32 query heads over 131072 tokens at d = 128 uses
 * 17.6 MB).  Limits and behaviour:
 *   - TQ_EWORKSPACE when tq_attention_workspace_bytes() of the arguments exceeds that maximum;
 *   - TQ_EUNSUPPORTED unless the device tables of pk and pv are already resident on the current
 *     device: any earlier call with the same parameters there builds them (the tq_encode that
 *     filled the caches does), and this entry point never builds them, since that allocates;
 *   - it calls no hipMalloc, hipFree or other allocating routine;
 *   - every call on one GPU uses that GPU's array, which keeps the last call's contents (every
 *     byte a call reads it has written first, so nothing needs clearing); calls that overlap on one
 *     GPU (other host threads, or other streams without ordering) race on it. */
int tq_decode_attention_noalloc(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype,
                                int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                                const void* packed_v, int64_t n_tokens, const int32_t* lengths,
                                float softmax_scale, void* out, tq_dtype out_dtype, void* stream);

/* Bytes of the device array tq_decode_attention_noalloc works in (the largest workspace it accepts). */
size_t tq_attention_noalloc_max_bytes(void);

/* Host-side copies of the tables the kernels use, for inspection and tests (no GPU call):
 * thresholds[2^b-1] and centroids[2^b] in fp64, signs[d] (±1) and S[m·d] (fp16 values as float)
 * of RNG head `head`.  Any output pointer may be NULL. */
int tq_host_tables(const tq_params* p, int32_t head, double* thresholds, double* centroids,
                   float* signs, float* S);

const char* tq_status_string(int status);
void tq_clear_cache(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
