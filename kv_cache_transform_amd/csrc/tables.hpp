// Host-side tables of the codec: random signs and Gaussian S (SplitMix64 + Box-Muller), the
// Lloyd-Max codebook of the rotated-coordinate density, and the derived lookup tables the gfx950
// kernels read (search grid, dequantisation LUTs, per-lane sign tables).
#pragma once
#include <cstdint>
#include <vector>

namespace tq {

// ---- random state: SplitMix64 (Steele, Lea, Flood 2014), counter form ------------------------
uint64_t mix64(uint64_t z);
uint64_t stream_key(uint64_t seed, uint32_t tag, uint32_t head);
// s_j = -1 iff bit 63 of word j (tag 1)
void head_signs(uint64_t seed, uint32_t head, int d, std::vector<float>& out);
// S[row][col] = fp16_rne(sqrt(-2 ln u1) cos(2 pi u2)) from words (2e, 2e+1), e = row*d + col (tag 2)
void gaussian_matrix_f16(uint64_t seed, uint32_t head, int m, int d, std::vector<uint16_t>& out);
// second signs s2 of the randomized Hadamard sketch: s2_j = -1 iff bit 63 of word j (tag 3)
void rht_signs(uint64_t seed, uint32_t head, int d, std::vector<float>& out);
// randomized Hadamard sketch S = H diag(s2): S[i][j] = (-1)^popcount(i & j) · s2_j; d x d entries
// of ±1 as fp16
void rht_matrix_f16(uint64_t seed, uint32_t head, int d, std::vector<uint16_t>& out);

// ---- Lloyd-Max codebook for f(x) ∝ (1-x^2)^((d-3)/2) on [-1,1] ---------------------------------
// thresholds[L-1], centroids[L] ascending, L = 2^b.  Returns 0 on success.
int lloyd_max(int d, int b, std::vector<double>& thresholds, std::vector<double>& centroids);

// ---- kernel-side derived tables ---------------------------------------------------------------
// Search grid in the affine domain u = y·G/2 + G/2 + 1 (y in [-1,1] -> u in [1, G+1]): the fp32
// thresholds thr_u = fp32(t·G/2 + G/2 + 1) are compared with the kernel's fp32 u.  Entry c (c = 0..G+2)
// covers u in [c, c+1) and holds {fp32 bits of the one threshold that can fall in the cell widened
// by a rounding margin (or +inf), count of thresholds below it}; for every u that lands in cell c,
// #{k : thr_u[k] <= u} == base + (u >= thr).  Cell 0 (NaN and rounding below -1) yields index 0.
struct Grid {
    int G = 0;
    std::vector<float> thr_u;
    std::vector<uint32_t> entries;  // 2 words per cell, G+3 cells
};
bool build_grid(const std::vector<double>& thr_y, Grid& out);

// Binade grid for b <= 4: u = 3 + kFqKappa·y lies in [2, 4) for every |y| <= 1, so bits 16..22 of
// u's fp32 pattern are a cell index c (128 cells of 1/64) and u >= thr compares as the integers.
// Entry c is E[c] = ((base_c + 1) << (32 - b)) - T_c (mod 2^32), with base_c the thresholds below
// the cell and T_c the bits of the one threshold inside it (or of the cell's upper end).  Then
// w = bits(u) + E[c] carries idx = #{k : thr_u[k] <= u} in its top b bits, and bits 16 .. 31 - b
// are all zero (u >= T_c) or all one (u < T_c), so the top byte of w is idx·2^(8-b) or
// idx·2^(8-b) + 2^(8-b) - 1.  Returns false if a cell would hold two thresholds.
constexpr double kFqKappa = 1.0 - 1.0 / 256.0;
bool build_fq_grid(const std::vector<double>& thr_y, int b, std::vector<uint32_t>& E);

// coordinates per dequantisation lookup for b bits
inline int lut_group(int b) { return (b == 1 || b == 2 || b == 4) ? 8 / b : ((b == 3 || b == 5 || b == 6) ? 2 : 1); }

uint16_t f32_to_f16_bits(float f);     // round to nearest even
uint16_t f64_to_f16_bits(double f);    // round to nearest even, one rounding
float f16_bits_to_f32(uint16_t h);

}  // namespace tq
