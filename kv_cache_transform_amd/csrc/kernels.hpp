// Kernel argument blocks and launcher declarations (host <-> .hip translation units).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Device-resident read-only tables for one (d, b, m, n_heads, seed); built on the host.
struct DevTables {
    int d = 0, b = 0, m = 0, n_heads = 0;
    uint64_t seed = 0;
    int sketch = 0;                    // TQ_SKETCH_GAUSSIAN or TQ_SKETCH_RHT
    int rotation = 0;                  // TQ_ROTATION_WHT or TQ_ROTATION_NONE (no sign flip, no WHT)
    int G = 0;                         // search grid cells
    const uint32_t* grid = nullptr;    // (G+2) x {thr fp32 bits, base}
    const uint32_t* fq_grid = nullptr; // binade grid (b <= 4): 128 entries E[c], or null
    const float* cent = nullptr;       // 2^b centroids (fp32)
    const float* cent_x1024 = nullptr; // 2^b centroids x 2^14 (fp32, exact scaling)
    const float* lut_f32 = nullptr;    // dequant LUT: 2^(P b) entries of P fp32 (P = lut_group(b))
    const _Float16* lut_f16 = nullptr; // same in fp16
    const _Float16* lut_hl = nullptr;  // per entry: P fp16 hi parts, then P fp16 lo parts of 2^12 x centroid
    // b = 4: the decode-attention's two LDS tables of 256-byte rows (2 x 256 x 64 words) as this
    // codec fills them: row e of table 0 = [fp16 value pair (c[e & 15], c[e >> 4]) x 32 | key hi
    // pair of byte e x 32], row e of table 1 = [key lo pair x 32 | zeros]; the kernel takes the
    // value words from the V codec's image and the rest from the K codec's; else null
    const uint32_t* attn_img = nullptr;
    const float* signs_slot = nullptr; // [head][4][d/4] ±1 of coordinate in_coord(d, s, g)
    const float* signs = nullptr;      // [head][d] ±1
    const float* signs2 = nullptr;     // [head][d] ±1 second signs of the RHT sketch (sketch = RHT only)
    const _Float16* S = nullptr;       // [head][m][d] fp16: Gaussian draws, or ±1 of H diag(s2) (m = d)
    void* blob = nullptr;              // single allocation owning all of the above
};

struct EncodeArgs {
    const void* x;           // [n_streams][n_tokens][d]
    uint8_t* packed;
    int64_t n_streams, n_tokens;
    int64_t cap, t0;         // the packed planes hold `cap` tokens per stream; x goes to [t0, t0 + n_tokens)
    int64_t off_idx, off_sketch, off_norm, off_rnorm;
    int64_t tiles_per_stream;  // ceil(n_tokens / 16)
    int64_t n_tiles;           // n_streams * tiles_per_stream
    int64_t tiles_per_wave;
    int64_t blocks_per_stream; // grid = n_streams * blocks_per_stream
    int64_t tiles_per_block;
    int grid_rep_log2;         // the search grid is held in LDS 2^grid_rep_log2 times (bank spread)
    DevTables t;
};

struct DecodeArgs {
    const uint8_t* packed;
    void* out;
    int64_t n_streams, n_tokens;
    int64_t off_idx, off_norm;
    int64_t off_sketch, off_rnorm;  // read only by the QJL-corrected decode
    int64_t tiles_per_stream, n_tiles, tiles_per_wave;
    int64_t blocks_per_stream, tiles_per_block;
    DevTables t;
};

// Query operands of the score products, written by qprep_kernel into the caller's workspace: per
// row r (a query of one stream), fp16 hi and lo parts of 2^e_r · q_scale · q_rot and of
// 2^e_r · p_scale · S q_rot (one power of two per row, chosen so the largest entry of the two lies in
// [2^13, 2^14): no fp16 overflow, and hi + lo hold every entry to ~2^-22 relative), and the row
// factor 2^-e_r that undoes the scaling.
struct QOps {
    _Float16* qh;           // [rows][d]
    _Float16* ql;           // [rows][d]
    _Float16* ph;           // [rows][m] (m > 0)
    _Float16* pl;           // [rows][m] (m > 0)
    float* rowf;            // [rows] 2^-e_r
};

struct QPrepArgs {
    const void* q;          // [n_rows][d], row r belongs to stream r / n_q_per_stream
    int q_bf16;
    int64_t n_rows;
    int n_q_per_stream;     // rows per stream (RNG head = stream % n_heads)
    QOps o;
    float q_scale, p_scale; // 1 for scores; attention folds its softmax scale (and the QJL factor) in
    DevTables t;
};

struct ScoresArgs {
    const uint8_t* packed;
    QOps o;                 // rows [n_streams][n_q]
    float* scores;          // [n_streams][n_q][n_tokens]
    int64_t n_streams, n_tokens;
    int n_q;
    int64_t off_idx, off_sketch, off_norm, off_rnorm;
    int64_t tiles_per_stream, n_tiles, tiles_per_wave;
    int64_t blocks_per_stream, tiles_per_block;
    DevTables t;
};

struct AttnArgs {
    const uint8_t* pk;       // packed K
    const uint8_t* pv;       // packed V
    QOps o;                  // rows [batch*n_q_heads]: q_rot (rotated with the K signs of its kv head)
                             // times scale_log2, S q_rot times scale_log2 sqrt(pi/2)/m
    float* part;             // [batch*n_kv][n_split][16 queries][d] rotated-domain partial sums
    float* part_ml;          // [batch*n_kv][n_split][16][2] running max (log2 units) and sum
    void* out;               // [batch][n_q_heads][d]
    int out_bf16;
    int64_t n_tokens;
    const int32_t* lens;     // [batch] valid tokens of each batch element's cache (clamped to
                             // [0, n_tokens]); null: all n_tokens
    int batch, n_q_heads, n_kv_heads, group;  // group = n_q_heads / n_kv_heads
    int n_split;
    int64_t tokens_per_split;
    float scale_log2;        // softmax scale * log2(e)
    int64_t k_off_idx, k_off_sketch, k_off_norm, k_off_rnorm;
    int64_t v_off_idx, v_off_norm;
    DevTables tk, tv;
    // the query prep inside the attention kernel (attention_fuses_qprep): each block computes its
    // stream's query operands from the raw queries q [batch][n_q_heads][d] (bf16 if q_bf16, else
    // fp32), scaled by q_scale and p_scale as the query prep kernel does; else o holds them
    int fused_q;
    const void* q;
    int q_bf16;
    float q_scale, p_scale;
};

// launchers: return hipSuccess or the launch error
hipError_t launch_encode(const EncodeArgs& a, bool x_bf16, int num_cus, hipStream_t s);
// keys and values of the same tokens in one launch (bf16 input); *fused = false: nothing launched
hipError_t launch_encode_kv(const EncodeArgs& ak, const EncodeArgs& av, int num_cus, hipStream_t s, bool* fused);
hipError_t launch_decode(const DecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s);
hipError_t launch_decode_qjl(const DecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s, bool* supported);
hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s);
hipError_t launch_scores(const ScoresArgs& a, int num_cus, hipStream_t s);
bool attention_supported(int d, int bk, int bv);
// whether launch_attention computes the query operands inside the attention kernel (every block's
// waves work on one stream, 4-bit keys and values, d <= 128, at most 8 query heads per kv head,
// m <= 128), so no query prep launch is needed
bool attention_fuses_qprep(const AttnArgs& a);
hipError_t launch_attention(const AttnArgs& a, int num_cus, hipStream_t s, bool* supported);

}  // namespace tq
