// Device tables and launchers of the SpectralQuant codec (calibrated eigenbasis, per-dimension
// Gaussian Lloyd-Max codebooks; "Ablation, Statistical Inference, and Validation for KV-Cache
// Compression", §2 "SpectralQuant").
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// Search-grid domain of a Gaussian codebook: u = z/σ in [-kSqRange, kSqRange] maps to
// u_grid = u·G/(2 kSqRange) + G/2 + 1 in [1, G+1]; outside it the cells clamp to 0 and G+2.
constexpr double kSqRange = 8.0;

struct SqDev {
    int d = 0, n_heads = 0, rec_words = 0;
    // encode: Uᵀ·2^8 as fp16 hi, lo in MFMA B-operand order [head][part][tile D/16][kstep D/32][lane][8]
    const _Float16* enc_b = nullptr;
    // encode: per (head, dimension k) {mul, add, meta, cmax}: u_grid = z·2^(8+sc)·mul... (see sq.hip)
    const float4* enc_desc = nullptr;
    const uint32_t* grids = nullptr;   // the grids of every width in use, 2 words per cell
    // decode: (U diag(σ))·2^e_h as fp16 hi, lo in MFMA A-operand order [head][part][tile][kstep][lane][8]
    const _Float16* dec_a = nullptr;
    const float* dec_scale = nullptr;  // [head] 2^-(e_h + 12)
    // field extraction per (head, kstep, lane part g): {first word | bit << 8, positions 1..4,
    // positions 5..7, widths}
    const uint4* fields = nullptr;
    const _Float16* cb_hl = nullptr;   // [width 0..8][256] (hi, lo) of c·2^12, 2 halves each
    const _Float16* cb_h = nullptr;    // [width 0..8][256] fp16 c
    const float* U32 = nullptr;        // [head][j][k] fp32
    const float* sigma = nullptr;      // [head][k]
    int lds_grid_words = 0;            // total words of `grids`
    // selective QJL sketch (m > 0): sketch rows over the first 32 dimensions (zero beyond d_eff)
    int m = 0;
    const _Float16* sk_b = nullptr;    // encode B operand [head][tile m/16][lane][8]: S[16ts + n][8g + i]
    const float* sk32 = nullptr;       // [head][64][32] fp32 S (rows >= m and columns >= d_eff zero)
    const int32_t* sk_off = nullptr;   // [head] bit offset of the sketch field (Σ_k b_k)
    const int32_t* deff = nullptr;     // [head] d_eff
    const float* cent32 = nullptr;     // [width 0..8][256] fp32 centroids
    const _Float16* pm1 = nullptr;     // [256][8] ±1 of a byte's bits, LSB first
    void* blob = nullptr;
};

struct SqEncodeArgs {
    SqDev t;
    const uint16_t* x;      // bf16 [streams][tokens][d]
    uint32_t* out;          // records [streams][tokens][rec_words]
    int64_t n_streams, n_tokens, tiles_per_stream;
    int64_t blocks_per_stream, tiles_per_block;
};

struct SqDecodeArgs {
    SqDev t;
    const uint32_t* in;
    void* out;              // fp32 or bf16 [streams][tokens][d]
    int64_t n_streams, n_tokens, tiles_per_stream;
    int64_t blocks_per_stream, tiles_per_block;
};

struct SqScoresArgs {
    SqDev t;
    const void* q;          // [streams][n_q][d] fp32 or bf16
    int q_bf16;
    const uint32_t* in;
    float* scores;          // [streams][n_q][tokens]
    _Float16* qp;           // workspace: [streams][nq_pad][d] fp16 of (Uᵀq ⊙ σ)·2^e_row
    float* qscale;          // workspace: [streams][nq_pad] 2^-e_row
    _Float16* pp;           // workspace with a sketch: [streams][nq_pad][64] fp16 of (S q_Z)·2^e'_row
    float* pscale;          // [streams][nq_pad] 2^-e'_row · sqrt(pi/2)/m (q_Z already carries qmul)
    float qmul;             // factor on every projected query (1 for scores; scale·log2 e for attention)
    _Float16* qplo = nullptr;  // [streams][nq_pad][d]: the fp16 remainder (q'·2^e - qp) of each entry
    _Float16* pplo = nullptr;  // with a sketch and not null: [streams][nq_pad][64] the fp16 remainder of pp
    int64_t n_streams, n_tokens, n_q, nq_pad, tiles_per_stream;
    int64_t blocks_per_stream, tiles_per_block;
};

struct SqAttnArgs {
    SqDev tk, tv;
    const _Float16* qp;     // [streams][16][d] fp16 projected queries (scaled by 2^e_row)
    const _Float16* qplo;   // [streams][16][d] their fp16 remainders (hi + lo = the fp32 value)
    const float* qscale;    // [streams][16] 2^-e_row
    const _Float16* pp;     // with a key sketch: [streams][16][64] fp16 S q_Z (scaled)
    const float* pscale;    // [streams][16]
    const uint32_t* kin;
    const uint32_t* vin;
    const int32_t* lens;    // [batch] or null
    float* part;            // [streams][n_split][16][d] unnormalised partial outputs in the V basis
    float* ml;              // [streams][n_split][16][2] running max (base 2) and sum
    void* out;              // [batch][hq][d]
    int out_bf16;
    int64_t n_streams, n_tokens, tps, n_split, hkv, hq, g;
};

hipError_t launch_sq_encode(const SqEncodeArgs& a, int num_cus, hipStream_t s);
hipError_t launch_sq_decode(const SqDecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s);
hipError_t launch_sq_scores(const SqScoresArgs& a, int num_cus, hipStream_t s);
hipError_t launch_sq_qprep(const SqScoresArgs& a, hipStream_t s);
hipError_t launch_sq_attention(const SqAttnArgs& a, hipStream_t s);

}  // namespace tq
