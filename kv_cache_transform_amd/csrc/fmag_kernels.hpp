// Device tables and launchers of the Fourier-magnitude codec ("Fourier Magnitude KV Cache
// Quantization", forum thread, "Method": FFT along head_dim, min-max magnitudes, kept or quantised
// phases, inverse FFT).
//
// Spectrum coordinates c = 0..d-1 (the order the DFT matrix's columns take): c < d/2 is Re X_c,
// c = d/2 is Re X_{d/2} (the Nyquist bin, in the slot of the always-zero Im X_0), c > d/2 is
// Im X_{c-d/2}.  With the MFMA output layout (lane n of a 16-lane row holds coordinate 16t + n) the
// real and imaginary parts of bin 16t' + n land in the same lane, in tiles t' and t' + d/32.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sq_kernels.hpp"

namespace tq {

struct FmDev {
    int d = 0, b = 0, p = 0, rec_words = 0;
    const _Float16* enc_b = nullptr;  // DFT·2^8 as fp16 hi, lo in MFMA B-operand order [part][t][s][lane][8]
    const _Float16* dec_a = nullptr;  // inverse DFT·2^e as fp16 hi, lo in A-operand order [part][t][s][lane][8]
    float dec_scale = 0.0f;           // 2^-e
    const float* cs = nullptr;        // [2^p][2] cos, sin of the phase levels (p <= 8)
    SqDev qprep;                      // U = the DFT matrix [j][c], σ = w_c/d: the query side of the scores
    const float* G32 = nullptr;       // [j][c] the weighted inverse real DFT in fp32 (attention combine)
    void* blob = nullptr;
};

struct FmEncodeArgs {
    FmDev t;
    const uint16_t* x;
    uint32_t* out;
    int64_t n_streams, n_tokens, tiles_per_stream;
    int64_t blocks_per_stream, tiles_per_block;
};

struct FmDecodeArgs {
    FmDev t;
    const uint32_t* in;
    void* out;
    int64_t n_streams, n_tokens, tiles_per_stream;
    int64_t blocks_per_stream, tiles_per_block;
};

struct FmScoresArgs {
    FmDev t;
    const _Float16* qp;     // [streams][nq_pad][d]
    const _Float16* qplo;   // [streams][nq_pad][d] fp16 remainders (qp + qplo = the fp32 value)
    const float* qscale;    // [streams][nq_pad]
    const uint32_t* in;
    float* scores;
    int64_t n_streams, n_tokens, n_q, nq_pad, tiles_per_stream;
    int64_t blocks_per_stream, tiles_per_block;
};

// decode-attention over Fmag K and V caches: one wave per (stream, split); the partial outputs stay
// in the spectrum domain (Σ_t p_t X̂_t), the combine merges the splits and applies the inverse DFT
struct FmAttnArgs {
    FmDev tk, tv;
    const _Float16* qp;     // [streams][16][d] projected queries (q' of the scores, times scale·log2 e)
    const _Float16* qplo;   // [streams][16][d] their fp16 remainders (hi + lo carry q' to about 2^-22)
    const float* qscale;    // [streams][16]
    const uint32_t* kin;
    const uint32_t* vin;
    const int32_t* lens;    // [batch] valid tokens, or null
    float* part;            // [streams·n_split][16][d] unnormalised spectrum-domain outputs
    float* ml;              // [streams·n_split][16][2] running max (base 2) and sum
    void* out;
    bool out_bf16;
    int64_t n_streams, n_tokens, tps, n_split;
    int hkv, hq, g;
};

hipError_t launch_fmag_encode(const FmEncodeArgs& a, int num_cus, hipStream_t s);
hipError_t launch_fmag_decode(const FmDecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s);
hipError_t launch_fmag_scores(const FmScoresArgs& a, int num_cus, hipStream_t s);
hipError_t launch_fmag_attention(const FmAttnArgs& a, hipStream_t s);
void fmag_clear_tables();

}  // namespace tq
