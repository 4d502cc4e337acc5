// Encode kernel ("Ablation, Statistical Inference, and Validation for KV-Cache Compression",
// §2 TurboQuant): per vector x, n = ||x||, y = H (x ⊙ s) / (sqrt(d) n), idx_j = #{i : t_i <= y_j},
// b-bit packing; with m > 0 also e = y - c[idx], ||e|| and sign(S e) (1-bit QJL of the residual).
//
// Three kernels: the search-grid encode (encode_kernel: any d, b and input type), the binade-grid
// encode of one tensor (encode_fq_kernel: bf16 input, b <= 4, d <= 128) and the binade-grid encode of
// the keys and values of the same tokens in one launch (encode_kv_kernel); the last two share the
// per-group code (fq_encode_group).
// Work split: one wave64 = 16 vectors x 4 parts (see common.hpp).  Waves walk a contiguous range of
// 16-vector tiles, so the per-head sign constants are reloaded only when the stream changes.
// Search: a uniform grid over y in [-1,1] held in LDS maps y to the one threshold that can lie in
// its cell plus the count of thresholds below; one compare finishes the search for any b.
// S·e: v_mfma_f32_16x16x32_f16 with the lane's own residual as the B operand (lane l = vector
// l%16, k-block l/16 matches the MFMA operand layout).  2^14 e (|2^14 e| < 2^15 always) is split
// into an fp16 part truncated toward zero and the fp16 rounding of the remainder, together exact
// to about 2^-22 relative; S is stored as fp16 values, so both products are exact and only the
// fp32 accumulation rounds.  z is then within ~1e-8 of the fp64 projection of the residual, far
// inside the 1e-6 band of a sign decision.
//
// Binade-grid variant (bf16 input, b <= 4, and for the sketch m <= 128): u = 3 + κ y lies in
// [2, 4), so the search grid is addressed by bits 16..22 of u's fp32 pattern.  One v_perm_b32 puts
// that byte next to the lane's copy offset (grid rows of 64 copies, one per lane: no bank
// conflicts), the entry E is added to u's bits, and the top bits of the sum are the index (see
// build_fq_grid): one v_alignbit packs it and one more v_perm_b32 addresses the lane's copy of
// its centroid, whose row is the sum's top byte.  The remaining tables (Hadamard tiles, S) sit in
// the rows of the centroid window that no top byte can reach.
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "tables.hpp"

namespace tq {

// LDS map of the binade-grid variant.  [0, 32 KiB): grid row c (c = 0..127) = 64 copies of E[c].
// From W = 32 KiB: the centroid window, 256 rows of 256 bytes addressed by the top byte of
// w = bits(u) + E; with R = 2^(8-b) only rows idx·R and idx·R + R - 1 can be addressed, and they
// hold 64 copies of 2^14 c[idx].  Rows idx·R + 1 .. idx·R + R - 2 hold 1 KiB pieces (four rows
// each, PPG per gap): the signed Hadamard tiles first, then S (or the randomized Hadamard tiles)
// in the order the MFMA A operand reads them.
template <int B>
struct FqLayout {
    static constexpr int W = 32768;
    static constexpr int R = 1 << (8 - B);
    static constexpr int PPG = (R - 2) / 4;
    static constexpr int cap = (1 << B) * PPG;
    static constexpr __host__ __device__ int piece(int p) { return W + ((p / PPG) * R + 1) * 256 + (p % PPG) * 1024; }
};
// LDS bytes of the binade-grid kernel: the whole centroid window with the sketch, else 64 KiB.  A
// grid or centroid address is at most 255·256 + 252 from its table's base whatever u is (a NaN
// input included), so every read stays inside the array.
template <int D, int B, bool QJL>
constexpr int fq_lds_bytes() { return QJL ? FqLayout<B>::W + 65536 : 65536; }

// Waves per block of the search-grid kernel: the sketch of bf16 input at d = 256 with S in LDS runs
// 8 waves (two per SIMD, 254 VGPRs) on one copy of S, which leaves no room for a second block;
// everything else runs 4.  (The binade-grid kernels below run one 12-wave block per CU.)
template <int D, bool QJL, bool BF16, bool S_LDS>
constexpr int enc_waves() {
    return (QJL && BF16 && S_LDS && D > 128) ? 8 : 4;
}
template <int D, bool QJL, bool BF16, bool S_LDS>
constexpr int enc_min_blocks() {
    return enc_waves<D, QJL, BF16, S_LDS>() == 8 ? 2
           : ((D > 128 && (QJL || !BF16)) || (QJL && !BF16) ? 1 : (D > 128 ? 2 : 3));
}

// The search-grid encode: any d, b and input type (the binade-grid kernels below serve bf16 input
// at b <= 4 and d <= 128).
template <int D, int B, bool QJL, bool BF16, bool S_LDS>
__global__ __launch_bounds__((64 * enc_waves<D, QJL, BF16, S_LDS>()), (enc_min_blocks<D, QJL, BF16, S_LDS>()))
void encode_kernel(EncodeArgs a) {
    constexpr int NWV = enc_waves<D, QJL, BF16, S_LDS>();
    constexpr int C = D / 4, R = D / 16, L = 1 << B;
    constexpr int NW = (C * B + 31) / 32;          // packed words per lane
    constexpr int CB = C * B / 8;                   // packed bytes per lane
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);
    constexpr int NG = (QJL && D <= 128 && !BF16) ? 2 : 1;   // 16-vector groups per pass (S-tile reuse)
    constexpr int KS = D / 32;                      // k-steps of 32 coordinates

    // ---- block = one stream's tile range; the RNG head is block-uniform -----------------------
    const int64_t st = blockIdx.x / a.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int m = a.t.m;

    extern __shared__ uint32_t lds[];
    const int G = a.t.G;
    // search grid, replicated 2^rl times with the copies interleaved per cell, so lanes that use
    // different copies read different banks: cell c of copy r = words 2 (c 2^rl + r) + {0, 1}
    const int rl = a.grid_rep_log2;
    const int ngw = (2 * (G + 3)) << rl;
    {
        for (int i = threadIdx.x; i < ((G + 3) << rl); i += blockDim.x) {
            const int c = i >> rl;
            lds[2 * i] = a.t.grid[2 * c];
            lds[2 * i + 1] = a.t.grid[2 * c + 1];
        }
    }
    float* lds_c = reinterpret_cast<float*>(lds + ngw);
    constexpr int NKB = D / 32;                     // K blocks of the 32-point transform
    constexpr int NAW = BF16 ? 2 * NKB * 64 * 4 : 0; // LDS words of the signed A tiles
    const int a_off = (ngw + L + 3) & ~3;
    u32x4* lds_A = reinterpret_cast<u32x4*>(lds + a_off);
    _Float16* lds_S = reinterpret_cast<_Float16*>(lds + a_off + NAW);
    if constexpr (QJL) {
        for (int i = threadIdx.x; i < L; i += blockDim.x) lds_c[i] = a.t.cent_x1024[i];
        if (S_LDS && !(BF16 && a.t.sketch == 1)) {
            // S in the order the MFMA A operand reads it (see the sketch loop): the 16-byte piece
            // of lane l for row tile tau and k-step k sits at piece index (tau KS + k) 64 + l, so
            // every A read is one contiguous 1 KiB wave access.  Lane l = rho + 16 gp reads row
            // (rho/4)(m/4) + 4 tau + rho%4, columns gp C + 8k .. +8.
            const u32x4* src = reinterpret_cast<const u32x4*>(a.t.S + (int64_t)head * m * D);
            u32x4* dst = reinterpret_cast<u32x4*>(lds_S);
            const int n16 = m * D / 8;             // 16-byte pieces
            const int mq = m >> 2;
            for (int i = threadIdx.x; i < n16; i += blockDim.x) {
                const int row = i / (D / 8), col = i - row * (D / 8);
                const int q = row / mq, rem = row - q * mq;
                const int tau = rem >> 2, rh = 4 * q + (rem & 3);
                const int gp = col / KS, k = col - gp * KS;
                dst[(tau * KS + k) * 64 + rh + 16 * gp] = src[i];
            }
        }
    }
    // bf16 input: the Hadamard transform over the 5 index bits {0,1,2, n-2, n-1} (n = log2 d) is a
    // dense 32-point block, run as v_mfma_f32_16x16x32_bf16 with the ±1 matrix as the A operand
    // (exact: ±1 and the bf16 inputs are exact, accumulation in fp32); the remaining middle bits
    // are radix-2 butterflies in registers.  Lane part g holds coordinates [g C, g C + C) both on
    // input (K block kb = 8 coordinates g C + 8 kb + jj) and on output (slot s = coordinate g C + s).
    // A tile (h, kb) of lane l holds row 4 mg + mi = l % 16, columns 8 (l/16) + jj:
    //   H[output (mg, h, mi)][input (l/16, jj)] * sign of input coordinate (l/16) C + 8 kb + jj,
    // with output coordinate bits {n-2,n-1} = mg, bit 2 = h, bits {0,1} = mi.  The random signs of
    // the head are folded in, so the tiles are built per block in LDS (one 16-byte entry per lane).
    // With the randomized Hadamard sketch (bf16 input), the same tiles with the second signs s2 and
    // ±1 in fp16 take the place of S: the sketch z = H (e ⊙ s2) is the same transform of the residual.
    if constexpr (BF16) {
        const bool rht = QJL && a.t.sketch == 1;
        for (int e = threadIdx.x; e < (rht ? 4 : 2) * NKB * 64; e += blockDim.x) {
            const int second = e >= 2 * NKB * 64;       // an RHT tile
            const int ee = second ? e - 2 * NKB * 64 : e;
            const int l = ee & 63, tile = ee >> 6, h = tile / NKB, kb = tile - h * NKB;
            const int lg = l >> 4, mi = l & 3, mg = (l >> 2) & 3;
            const float* sh = (second ? a.t.signs2 : a.t.signs) + (int64_t)head * D + lg * C + 8 * kb;
            const uint32_t one = second ? 0x3c00u : 0x3f80u;   // fp16 / bf16 +1
            u32x4 wv;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t w2 = 0u;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int jj = 2 * t + q;
                    const uint32_t par = (uint32_t)((__builtin_popcount(mi & jj & 3) + h * (jj >> 2) +
                                                     __builtin_popcount(mg & lg)) & 1) ^ (f2u(sh[jj]) >> 31);
                    w2 |= (one | (par << 15)) << (16 * q);
                }
                wv[t] = w2;
            }
            if (second) reinterpret_cast<u32x4*>(lds_S)[ee] = wv;
            else lds_A[e] = wv;
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int v = lane & 15, g = lane >> 4;
    const int wave = wave_id();
    const bool plain = a.t.rotation == 1;          // Plain-KV: no sign flip, no WHT
    const float gA = 0.5f * (float)G;
    const float gB = 0.5f * (float)G + 1.0f;       // entry 0 is a guard cell

    float sg[BF16 ? 1 : C];
    if constexpr (!BF16) {
        const float* ss = a.t.signs_slot + ((int64_t)head * 4 + g) * C;
#pragma unroll
        for (int s = 0; s < C; ++s) sg[s] = ss[s];
    }
    // QJL A-operand rows: MFMA row slot rho of tile tau is sketch row (rho/4)*(m/4) + 4 tau + rho%4,
    // so lane part g collects rows [g m/4, (g+1) m/4), a contiguous bit chunk of the sketch.
    const int rho = lane & 15;
    const int row_base = (rho >> 2) * (m >> 2) + (rho & 3);
    const uint32_t goff = (uint32_t)(lane & ((1 << rl) - 1)) << 3;   // byte offset of the lane's grid copy

    // raw input words of one 16-vector group: bf16 = the lane's C contiguous coordinates; fp32 =
    // runs of R coordinates in the i(s, g) order of the butterfly network (see common.hpp)
    constexpr int NIW = BF16 ? C / 2 : C;
    auto load_group = [&](uint32_t (&w)[NIW], int64_t tile) {
        const int64_t tok = tile * 16 + v;
        const bool valid = tile < tb1 && tok < a.n_tokens;
        const int64_t vec = st * a.n_tokens + (valid ? tok : 0);
        if constexpr (BF16) {
            // a vector past the end reads token 0 of the stream (in bounds); nothing of it is stored,
            // and every MFMA column / 4-lane reduction stays within one vector
            const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x) + vec * (int64_t)(2 * D) + 2 * g * C;
            load_bytes<2 * C, 16>(base, w);
        } else {
            constexpr int RB = 4 * R;                     // bytes per run
            constexpr int RA = cmin(pow2_align(RB), 16);
            if (plain) {                                  // no rotation: coordinates g C .. g C + C - 1
                if (valid) load_bytes<4 * C, 16>(reinterpret_cast<const uint8_t*>(a.x) + vec * (int64_t)(4 * D) + 4 * g * C, w);
                else {
#pragma unroll
                    for (int k = 0; k < NIW; ++k) w[k] = 0u;
                }
                return;
            }
            const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x) + vec * (int64_t)(4 * D) + 4 * g * R;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (valid) load_bytes<RB, RA>(base + r * D, &w[r * (NIW / 4)]);
                else {
#pragma unroll
                    for (int k = 0; k < NIW / 4; ++k) w[r * (NIW / 4) + k] = 0u;
                }
            }
        }
    };
    uint32_t nxt[NG][NIW];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) load_group(nxt[gi], tb0 + wave * NG + gi);

#pragma unroll 1
    for (int64_t t = tb0 + wave * NG; t < tb1; t += NWV * NG) {
        // keep the LDS operand tables in LDS (re-read per pass) instead of pinned in registers
        asm volatile("" ::: "memory");
        half8 bh[NG][QJL ? C / 8 : 1], bl[NG][QJL ? C / 8 : 1];
        float e2v[NG];
        bool validv[NG];
        int64_t vecv[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int64_t tok = (t + gi) * 16 + v;
            const bool valid = (t + gi) < tb1 && tok < a.n_tokens;
            // packed record of this vector: token t0 + tok of a cache of `cap` tokens per stream
            const int64_t vec = st * a.cap + a.t0 + (valid ? tok : 0);
            validv[gi] = valid;
            vecv[gi] = vec;

            // ---- sign, first butterfly stage, norm ----------------------------------------------
            float x[C];
            float n2 = 0.0f;
            uint32_t (&w)[NIW] = nxt[gi];
            if constexpr (BF16) {
#pragma unroll
                for (int k = 0; k < C / 2; ++k) {
                    const bf16x2 wv = __builtin_bit_cast(bf16x2, w[k]);
                    n2 = __builtin_amdgcn_fdot2_f32_bf16(wv, wv, n2, false);
                }
                if (plain) {
                    // no rotation: slot s is coordinate g C + s itself
#pragma unroll
                    for (int k = 0; k < C / 2; ++k) {
                        x[2 * k] = u2f(w[k] << 16);
                        x[2 * k + 1] = u2f(w[k] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const bf16x8 Bv = __builtin_bit_cast(bf16x8, u32x4{w[4 * kb], w[4 * kb + 1], w[4 * kb + 2], w[4 * kb + 3]});
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const u32x4 At = lds_A[(h * NKB + kb) * 64 + lane];
                            const floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, At), Bv,
                                floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                            for (int i = 0; i < 4; ++i) x[8 * kb + 4 * h + i] = r[i];
                        }
                    }
                }
                // last reads of the raw words: the next pass's loads may reuse their registers
#pragma unroll
                for (int k = 0; k < NIW; ++k) asm volatile("" ::"v"(w[k]) : "memory");
                asm volatile("" ::"v"(n2) : "memory");
                if (t + NWV * NG < tb1) load_group(nxt[gi], t + NWV * NG + gi);
                if (!plain) fwht_slots<C, 8>(x);
            } else {
#pragma unroll
                for (int s = 0; s < C; ++s) {
                    const float xv = u2f(w[s]);
                    n2 = fmaf(xv, xv, n2);
                    x[s] = plain ? xv : xv * sg[s];
                }
                if (t + NWV * NG < tb1) load_group(nxt[gi], t + NWV * NG + gi);
                if (!plain) {
                    fwht_slots<C, 1>(x);
                    fwht_cross<C>(x);
                }
            }
            n2 = sum4(n2);
            // hardware square root and reciprocal square root (about 1 ulp: y moves by ~1e-7, far
            // inside the 1e-6 decision bands); a denormal n² keeps the exact forms
            float n, sc;
            if (n2 >= 0x1p-126f) {
                n = __builtin_amdgcn_sqrtf(n2);
                sc = (plain ? 1.0f : kInvSqrtD) * __builtin_amdgcn_rsqf(n2);
            } else {
                n = sqrtf(n2);
                sc = n > 0.0f ? (plain ? 1.0f : kInvSqrtD) / n : 0.0f;
            }
            const float sA = sc * gA;
            const float sE = sc * 16384.0f;

            // ---- scalar quantiser + pack (and the scaled residual for QJL) ----------------------
            // The grid lives in the affine domain u = y G/2 + G/2 + 1; thresholds are stored there.
            uint32_t pk[NW];
#pragma unroll
            for (int k = 0; k < NW; ++k) pk[k] = 0u;
            float e2 = 0.0f;
#pragma unroll
            for (int s = 0; s < C; ++s) {
                const float u = fmaf(x[s], sA, gB);
                const uint32_t cell = (uint32_t)u;
                const u32x2 ent = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(lds) + ((cell << (3 + rl)) + goff));
                const uint32_t thr = ent[0], base = ent[1];
                const uint32_t idx = base + (u >= u2f(thr) ? 1u : 0u);
                put_bits<B>(pk, s * B, idx);
                if constexpr (QJL) {
                    const float e = fmaf(x[s], sE, -lds_c[idx]);  // 2^14 (y - c[idx])
                    x[s] = e;
                    e2 = fmaf(e, e, e2);
                }
            }
            if (valid) {
                store_bytes<CB, CA>(a.packed + a.off_idx + vec * (int64_t)(D * B / 8) + g * CB, pk);
                if (g == 0) *reinterpret_cast<_Float16*>(a.packed + a.off_norm + vec * 2) = (_Float16)n;
            }
            if constexpr (QJL) {
                e2v[gi] = e2;
                // B operands: lane's residual slots [8k, 8k+8) for k-step k, as hi + lo fp16 parts
#pragma unroll
                for (int k = 0; k < C / 8; ++k) {
                    u32x4 hv, lv;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float e0 = x[8 * k + 2 * u], e1 = x[8 * k + 2 * u + 1];
                        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
                        hv[u] = h;
                        lv[u] = sub_f16pair_from_f32(h, e0, e1);
                    }
                    bh[gi][k] = __builtin_bit_cast(half8, hv);
                    bl[gi][k] = __builtin_bit_cast(half8, lv);
                }
            }
        }

        if constexpr (QJL && BF16) {
          if (a.t.sketch == 1) {
            // randomized Hadamard sketch z = H (e ⊙ s2) (m = d): the rotation's 32-point block on
            // fp16 MFMA with the s2 tiles as A and the residual's hi then lo parts as B, then
            // the middle-bit butterflies; slot p of part g is sketch row g C + p, so the part's C
            // bits are its z slots in order (one byte per 8 slots via alignbit, inverted: z >= 0)
            const u32x4* lds_A2 = reinterpret_cast<const u32x4*>(lds_S);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                float z[C];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const half8 A = __builtin_bit_cast(half8, lds_A2[(h * NKB + kb) * 64 + lane]);
                        floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[gi][kb], floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[gi][kb], r, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) z[8 * kb + 4 * h + i] = r[i];
                    }
                fwht_slots<C, 8>(z);
                uint8_t* dst = a.packed + a.off_sketch + vecv[gi] * (int64_t)(D / 8) + g * (C / 8);
#pragma unroll
                for (int w = 0; w < (C + 31) / 32; ++w) {
                    constexpr int NBY = C < 32 ? C / 8 : 4;      // bytes per word
                    uint32_t by[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int j = 0; j < NBY; ++j)
#pragma unroll
                        for (int p = 8 * j + 7; p >= 8 * j; --p) by[j] = __builtin_amdgcn_alignbit(by[j], f2u(z[32 * w + p]), 31);
                    const uint32_t bw = ~((((by[3] << 8) | by[2]) << 16) | ((by[1] << 8) | by[0]));
                    if (validv[gi]) {
                        if constexpr (NBY == 4) *reinterpret_cast<uint32_t*>(dst + 4 * w) = bw;
                        else *reinterpret_cast<uint16_t*>(dst + 4 * w) = (uint16_t)bw;
                    }
                }
            }
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const float e2 = sum4(e2v[gi]);
                if (validv[gi] && g == 0) {
                    const _Float16 r16 = (_Float16)(sqrtf(e2) * (1.0f / 16384.0f));
                    *reinterpret_cast<_Float16*>(a.packed + a.off_rnorm + vecv[gi] * 2) = r16;
                }
            }
            continue;
          }
        }
        if constexpr (QJL) {
            const _Float16* Sg = S_LDS ? (lds_S + 8 * lane) : (a.t.S + ((int64_t)head * m + row_base) * D + g * C);
            // sketch bits of lane part g: rows [g m/4, (g+1) m/4), 32 per word; tile tt of a word
            // holds rows 4 tt + i (bit 4 tt + i).  The products run k-step outer, tile inner, so
            // the 8 tiles' accumulations are independent MFMA chains and the S reads of later steps
            // can be in flight meanwhile.  Bits are gathered as one byte per tile pair (alignbit
            // shifts each sign in at bit 0), the bytes joined, and the word inverted (z >= 0).
            // Full words run branch-free; a trailing partial word (m/4 not a multiple of 32) has
            // nt < 8 tiles.
            auto sketch_word = [&](auto wb, int nt, auto full) {
                constexpr bool FULL = decltype(full)::value;
                const int tau0 = wb >> 2;
                uint32_t by[NG][4];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {                // tiles 4 hf .. 4 hf + 3: bytes 2 hf, 2 hf + 1
                    floatx4 acc[NG][4];
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                        for (int tl = 0; tl < 4; ++tl) acc[gi][tl] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KS; ++k) {
#pragma unroll
                        for (int tl = 0; tl < 4; ++tl) {
                            const int tt = 4 * hf + tl;
                            if (FULL || tt < nt) {
                                const int tau = tau0 + tt;
                                const half8 A = *reinterpret_cast<const half8*>(S_LDS ? Sg + (tau * KS + k) * 512 : Sg + 4 * tau * D + 8 * k);
#pragma unroll
                                for (int gi = 0; gi < NG; ++gi) {
                                    acc[gi][tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[gi][k], acc[gi][tl], 0, 0, 0);
                                    acc[gi][tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[gi][k], acc[gi][tl], 0, 0, 0);
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                        for (int j = 2 * hf; j < 2 * hf + 2; ++j) {
                            by[gi][j] = 0u;
#pragma unroll
                            for (int tt = 2 * j + 1; tt >= 2 * j; --tt)
                                if (FULL || tt < nt)
#pragma unroll
                                    for (int i = 3; i >= 0; --i)
                                        by[gi][j] = __builtin_amdgcn_alignbit(by[gi][j], f2u(acc[gi][tt - 4 * hf][i]), 31);
                        }
                }
                if constexpr (FULL && NG == 1) {
                    // issue order: the first kPD S reads, then per step its two MFMAs and the read
                    // kPD steps ahead, so each read has kPD steps of matrix work to land
                    constexpr int kPD = 4;
                    __builtin_amdgcn_sched_group_barrier(0x100, kPD, 0);
#pragma unroll
                    for (int p = 0; p < 8 * KS; ++p) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                        if (p + kPD < 8 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
                const int nb = FULL ? 4 : (nt >> 1);          // bytes in this word
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const uint32_t bw = ~((((by[gi][3] << 8) | by[gi][2]) << 16) | ((by[gi][1] << 8) | by[gi][0]));
                    if (validv[gi]) {
                        uint8_t* dst = a.packed + a.off_sketch + vecv[gi] * (int64_t)(m / 8) + g * (m / 32) + (wb >> 3);
                        if (FULL && (m & 127) == 0) *reinterpret_cast<uint32_t*>(dst) = bw;
                        else if (nb == 2 && (m & 63) == 0) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bw;
                        else for (int q = 0; q < nb; ++q) dst[q] = (uint8_t)(bw >> (8 * q));
                    }
                }
            };
            const int nbits = m >> 2;
            for (int wb = 0; wb + 32 <= nbits; wb += 32) sketch_word(wb, 8, std::true_type{});
            if (nbits & 31) sketch_word(nbits & ~31, (nbits & 31) >> 2, std::false_type{});
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const float e2 = sum4(e2v[gi]);
                if (validv[gi] && g == 0) {
                    const _Float16 r16 = (_Float16)(sqrtf(e2) * (1.0f / 16384.0f));
                    *reinterpret_cast<_Float16*>(a.packed + a.off_rnorm + vecv[gi] * 2) = r16;
                }
            }
        }
    }
}

// resident blocks per CU of kernel k at `threads` per block and `lds` bytes of dynamic LDS (cached
// per kernel and size)
static int blocks_per_cu(const void* k, size_t lds, int threads) {
    static std::mutex mu;
    static std::map<std::pair<const void*, size_t>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({k, lds});
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, threads, lds) != hipSuccess || n < 1) n = 1;
    cache[{k, lds}] = n;
    return n;
}

// ---------------------------------------------------------------------------------------------
// Keys and values of the same tokens in one launch (bf16 input, the same d <= 128 and b <= 4 for
// both, so one codebook and one binade grid; values without a sketch).  The QJL key encode is bound
// by VALU issue (the quantiser's chain per coordinate plus the sketch products) while the value
// encode is bound by HBM, so each wave encodes the key group and then the value group of the same
// 16 tokens: the values' loads and stores stream while the keys' arithmetic holds the SIMD.  The
// arithmetic per vector is the single-tensor binade-grid kernel's, step for step, so the records
// are identical to two separate encodes.  LDS: the shared grid, the keys' centroid rows, then in
// the window pieces the keys' signed Hadamard tiles, their S (or randomized Hadamard tiles) and
// the values' signed Hadamard tiles.

// one tensor's buffers over the block's stream (as in the binade-grid kernel: each exactly as long
// as the stream's part, so a lane past the last token reads zeros and its stores are dropped)
struct FqBufs {
    __amdgpu_buffer_rsrc_t rx, rid, rnm, rsk, rrn;
};

// One 16-vector group of one tensor: w holds the lane's raw bf16 words of tile t and receives the
// loads of tile t_next (issued as soon as w is consumed; skipped when t_next >= tb1).  pA is the
// first window piece of the tensor's signed Hadamard tiles, pS that of its S / randomized tiles.
template <int D, int B, bool QJL>
__device__ __forceinline__ void fq_encode_group(const uint8_t* ldsb, int pA, int pS, bool rht, bool plain, int m,
                                                const FqBufs& R, uint32_t (&w)[D / 8], int64_t t, int64_t t_next,
                                                int64_t tb1, int64_t n_tokens, int lane) {
    using FL = FqLayout<B>;
    constexpr int C = D / 4, NKB = D / 32, KS = D / 32;
    constexpr int NW = (C * B + 31) / 32, CB = C * B / 8, CA = cmin(pow2_align(CB), 16);
    constexpr float kInvSqrtD = D == 64 ? 0.125f : 0.08838834764831845f;
    const int v = lane & 15, g = lane >> 4;
    const uint32_t lane4 = 4u * (uint32_t)lane;
    const int64_t tok = t * 16 + v;
    const bool valid = t < tb1 && tok < n_tokens;
    const uint32_t tk = (uint32_t)tok;

    // sign flip + 32-point block on bf16 MFMA, then the middle bits in registers (Plain-KV: slot s
    // is coordinate g C + s itself); the norm
    float x[C];
    float n2 = 0.0f;
#pragma unroll
    for (int k = 0; k < C / 2; ++k) {
        const bf16x2 wv = __builtin_bit_cast(bf16x2, w[k]);
        n2 = __builtin_amdgcn_fdot2_f32_bf16(wv, wv, n2, false);
    }
    if (plain) {
#pragma unroll
        for (int k = 0; k < C / 2; ++k) {
            x[2 * k] = u2f(w[k] << 16);
            x[2 * k + 1] = u2f(w[k] & 0xffff0000u);
        }
    } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 Bv = __builtin_bit_cast(bf16x8, u32x4{w[4 * kb], w[4 * kb + 1], w[4 * kb + 2], w[4 * kb + 3]});
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 At = *reinterpret_cast<const u32x4*>(ldsb + FL::piece(pA + h * NKB + kb) + 16 * lane);
            const floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, At), Bv,
                                                                     floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[8 * kb + 4 * h + i] = r[i];
        }
    }
    }
#pragma unroll
    for (int k = 0; k < D / 8; ++k) asm volatile("" ::"v"(w[k]) : "memory");
    asm volatile("" ::"v"(n2) : "memory");
    if (t_next < tb1) bload<2 * C, 16>(R.rx, (uint32_t)(t_next * 16 + v) * (2 * D) + 2 * g * C, 0u, w);
    if (!plain) fwht_slots<C, 8>(x);
    n2 = sum4(n2);
    // hardware square root and reciprocal square root (about 1 ulp: y moves by ~1e-7, far inside
    // the 1e-6 decision bands); a denormal n² keeps the exact forms
    const float inv_sqrt_d = plain ? 1.0f : kInvSqrtD;
    float n, sc;
    if (n2 >= 0x1p-126f) {
        n = __builtin_amdgcn_sqrtf(n2);
        sc = inv_sqrt_d * __builtin_amdgcn_rsqf(n2);
    } else {
        n = sqrtf(n2);
        sc = n > 0.0f ? inv_sqrt_d / n : 0.0f;
    }
    const float sE = sc * 16384.0f;

    // quantise + pack (slots in descending order, so alignbit leaves the lowest slot in the low bits)
    uint32_t pk[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) pk[k] = 0u;
    float e2 = 0.0f;
    const float sU = sc * (float)kFqKappa;
#pragma unroll
    for (int s = C - 1; s >= 0; --s) {
        const float u = fmaf(x[s], sU, 3.0f);
        const uint32_t ga = __builtin_amdgcn_perm(f2u(u), lane4, 0x0c0c0600u);
        const uint32_t wq = f2u(u) + *reinterpret_cast<const uint32_t*>(ldsb + ga);
        if constexpr (B == 3) put_bits<B>(pk, s * B, wq >> 29);
        else pk[(s * B) >> 5] = __builtin_amdgcn_alignbit(pk[(s * B) >> 5], wq, 32 - B);
        if constexpr (QJL) {
            const uint32_t ca = __builtin_amdgcn_perm(wq, lane4, 0x0c0c0700u);
            x[s] = fmaf(x[s], sE, -*reinterpret_cast<const float*>(ldsb + FL::W + ca));
            e2 = fmaf(x[s], x[s], e2);
        }
    }
    if (valid) {
        bstore<CB, CA>(R.rid, tk * (D * B / 8) + g * CB, 0u, pk);
        if (g == 0) __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)n), R.rnm, tk * 2u, 0u, 0);
    }
    if constexpr (QJL) {
        // the residual 2^14 e as fp16 hi (truncated) + lo parts: the B operands of S·e
        half8 bh[C / 8], bl[C / 8];
#pragma unroll
        for (int k = 0; k < C / 8; ++k) {
            u32x4 hv, lv;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float e0 = x[8 * k + 2 * u], e1 = x[8 * k + 2 * u + 1];
                const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
                hv[u] = h;
                lv[u] = sub_f16pair_from_f32(h, e0, e1);
            }
            bh[k] = __builtin_bit_cast(half8, hv);
            bl[k] = __builtin_bit_cast(half8, lv);
        }
        if (rht) {
            // z = H (e ⊙ s2): the 32-point block with the s2 tiles on fp16 MFMA, hi then lo parts, and
            // the middle bits; slot p of part g is sketch row g C + p (one byte per 8 slots, inverted)
            float z[C];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const half8 A = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(ldsb + FL::piece(pS + h * NKB + kb) + 16 * lane));
                    floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[kb], floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[kb], r, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[8 * kb + 4 * h + i] = r[i];
                }
            fwht_slots<C, 8>(z);
#pragma unroll
            for (int wd = 0; wd < (C + 31) / 32; ++wd) {
                constexpr int NBY = C < 32 ? C / 8 : 4;
                uint32_t by[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int j = 0; j < NBY; ++j)
#pragma unroll
                    for (int p = 8 * j + 7; p >= 8 * j; --p) by[j] = __builtin_amdgcn_alignbit(by[j], f2u(z[32 * wd + p]), 31);
                const uint32_t bw = ~((((by[3] << 8) | by[2]) << 16) | ((by[1] << 8) | by[0]));
                if (valid) {
                    const uint32_t o = tk * (D / 8) + g * (C / 8) + 4 * wd;
                    if constexpr (NBY == 4) __builtin_amdgcn_raw_buffer_store_b32(bw, R.rsk, o, 0u, 0);
                    else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bw, R.rsk, o, 0u, 0);
                }
            }
        } else {
            // Gaussian S (m <= 128: one sketch word per lane part, rows [g m/4, (g+1) m/4)); the products
            // run k-step outer and row tile inner, and the S reads are issued ahead of their MFMAs
            auto word = [&](int nt, auto full) {
                constexpr bool FULL = decltype(full)::value;
                uint32_t by[4];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    floatx4 acc[4];
#pragma unroll
                    for (int tl = 0; tl < 4; ++tl) acc[tl] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KS; ++k)
#pragma unroll
                        for (int tl = 0; tl < 4; ++tl) {
                            const int tt = 4 * hf + tl;
                            if (FULL || tt < nt) {
                                const half8 A = *reinterpret_cast<const half8*>(ldsb + FL::piece(pS + tt * KS + k) + 16 * lane);
                                acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[k], acc[tl], 0, 0, 0);
                                acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[k], acc[tl], 0, 0, 0);
                            }
                        }
#pragma unroll
                    for (int j = 2 * hf; j < 2 * hf + 2; ++j) {
                        by[j] = 0u;
#pragma unroll
                        for (int tt = 2 * j + 1; tt >= 2 * j; --tt)
                            if (FULL || tt < nt)
#pragma unroll
                                for (int i = 3; i >= 0; --i)
                                    by[j] = __builtin_amdgcn_alignbit(by[j], f2u(acc[tt - 4 * hf][i]), 31);
                    }
                }
                if constexpr (FULL) {
                    constexpr int kPD = 4;
                    __builtin_amdgcn_sched_group_barrier(0x100, kPD, 0);
#pragma unroll
                    for (int p = 0; p < 8 * KS; ++p) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                        if (p + kPD < 8 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
                const int nb = FULL ? 4 : (nt >> 1);
                const uint32_t bw = ~((((by[3] << 8) | by[2]) << 16) | ((by[1] << 8) | by[0]));
                if (valid) {
                    const uint32_t o = tk * (uint32_t)(m / 8) + (uint32_t)(g * (m / 32));
                    if (FULL && (m & 127) == 0) __builtin_amdgcn_raw_buffer_store_b32(bw, R.rsk, o, 0u, 0);
                    else if (nb == 2 && (m & 63) == 0) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bw, R.rsk, o, 0u, 0);
                    else for (int q = 0; q < nb; ++q) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(bw >> (8 * q)), R.rsk, o + q, 0u, 0);
                }
            };
            const int nbits = m >> 2;
            if (nbits == 32) word(8, std::true_type{});
            else word(nbits >> 2, std::false_type{});
        }
        const float e2s = sum4(e2);
        if (valid && g == 0) {
            const _Float16 r16 = (_Float16)(sqrtf(e2s) * (1.0f / 16384.0f));
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, r16), R.rrn, tk * 2u, 0u, 0);
        }
    }
}

// LDS pieces of the signed Hadamard tiles of one head's signs (bf16 ±1, the 32-point block's A
// operand, as the binade-grid kernel builds them) at pieces pA .. pA + 2 D/32 - 1; `second` builds
// the randomized-Hadamard tiles instead (s2, fp16 ±1)
template <int D, int B>
__device__ __forceinline__ void fq_stage_hadamard(uint8_t* ldsb, int pA, const float* signs, bool second, int tid, int nth) {
    using FL = FqLayout<B>;
    constexpr int C = D / 4, NKB = D / 32;
    for (int e = tid; e < 2 * NKB * 64; e += nth) {
        const int l = e & 63, tile = e >> 6, h = tile / NKB, kb = tile - h * NKB;
        const int lg = l >> 4, mi = l & 3, mg = (l >> 2) & 3;
        const float* sh = signs + lg * C + 8 * kb;
        const uint32_t one = second ? 0x3c00u : 0x3f80u;   // fp16 / bf16 +1
        u32x4 wv;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t w2 = 0u;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int jj = 2 * t + q;
                const uint32_t par = (uint32_t)((__builtin_popcount(mi & jj & 3) + h * (jj >> 2) +
                                                 __builtin_popcount(mg & lg)) & 1) ^ (f2u(sh[jj]) >> 31);
                w2 |= (one | (par << 15)) << (16 * q);
            }
            wv[t] = w2;
        }
        *reinterpret_cast<u32x4*>(ldsb + FL::piece(pA + tile) + 16 * l) = wv;
    }
}

// The binade-grid tables of one key or value codec (as both binade-grid kernels stage them): grid
// row c = 64 copies of E[c]; with the sketch the centroid rows (64 copies of 2^14 c[idx] in rows
// idx·R and idx·R + R - 1) and, for the Gaussian sketch (m <= 128 here), S in the MFMA A-operand
// order at window pieces pS onwards: lane l = rho + 16 gp of row tile tau, k-step k reads row
// (rho/4)(m/4) + 4 tau + rho%4, columns gp C + 8k .. +8.  Every global load is issued before any
// LDS store (compile-time trip counts), so the prologue waits on memory once.
constexpr int kFqWaves = 12;                      // waves per block of the binade-grid kernels
template <int D, int B, bool QJL>
__device__ __forceinline__ void fq_stage_tables(uint8_t* ldsb, const DevTables& t, int head, int m, bool rht, int pS,
                                                int tid) {
    using FL = FqLayout<B>;
    constexpr int NTH = 64 * kFqWaves, KS = D / 32;
    constexpr int NGI = (128 * 64 + NTH - 1) / NTH;
    constexpr int NCE = 2 * (1 << B) * 64;         // centroid-row words
    constexpr int NCI = QJL ? (NCE + NTH - 1) / NTH : 1;
    constexpr int NSI = QJL ? (128 * D / 8 + NTH - 1) / NTH : 1;
    uint32_t* const ldsw = reinterpret_cast<uint32_t*>(ldsb);
    uint32_t gv[NGI], cv[NCI];
    u32x4 sv[NSI];
#pragma unroll
    for (int j = 0; j < NGI; ++j) {
        const int i = tid + j * NTH;
        gv[j] = t.fq_grid[(i < 128 * 64 ? i : 0) >> 6];
    }
    const int n16 = QJL && !rht ? m * D / 8 : 0;   // 16-byte pieces of S
    if constexpr (QJL) {
#pragma unroll
        for (int j = 0; j < NCI; ++j) {
            const int i = tid + j * NTH;
            cv[j] = f2u(t.cent_x1024[i < NCE ? (i >> 7) : 0]);
        }
        if (n16 > 0) {
            const u32x4* src = reinterpret_cast<const u32x4*>(t.S + (int64_t)head * m * D);
#pragma unroll
            for (int j = 0; j < NSI; ++j) {
                const int i = tid + j * NTH;
                if (i < n16) sv[j] = src[i];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NGI; ++j) {
        const int i = tid + j * NTH;
        if (i < 128 * 64) ldsw[i] = gv[j];
    }
    if constexpr (QJL) {
#pragma unroll
        for (int j = 0; j < NCI; ++j) {
            const int i = tid + j * NTH;
            if (i < NCE) {
                const int r2 = i >> 6, idx = r2 >> 1, row = idx * FL::R + ((r2 & 1) ? FL::R - 1 : 0);
                ldsw[(FL::W + row * 256) / 4 + (i & 63)] = cv[j];
            }
        }
        if (n16 > 0) {
            const int mq = m >> 2;
#pragma unroll
            for (int j = 0; j < NSI; ++j) {
                const int i = tid + j * NTH;
                if (i < n16) {
                    const int row = i / (D / 8), col = i - row * (D / 8);
                    const int q = row / mq, rem = row - q * mq;
                    const int tau = rem >> 2, rh = 4 * q + (rem & 3);
                    const int gp = col / KS, k = col - gp * KS;
                    *reinterpret_cast<u32x4*>(ldsb + FL::piece(pS + tau * KS + k) + 16 * (rh + 16 * gp)) = sv[j];
                }
            }
        }
    }
}

// raw buffers over stream st's input and its tokens' record planes, each exactly as long as the
// stream's part (the launchers keep them below 2^31 bytes)
template <int D, int B>
__device__ __forceinline__ FqBufs fq_bufs(const EncodeArgs& a, int64_t st, bool qjl) {
    FqBufs R;
    const int64_t rec0 = st * a.cap + a.t0;
    R.rx = buffer_rsrc(reinterpret_cast<const uint8_t*>(a.x) + st * a.n_tokens * (int64_t)(2 * D), (int)(a.n_tokens * 2 * D));
    R.rid = buffer_rsrc(a.packed + a.off_idx + rec0 * (int64_t)(D * B / 8), (int)(a.n_tokens * (D * B / 8)));
    R.rnm = buffer_rsrc(a.packed + a.off_norm + rec0 * 2, (int)(a.n_tokens * 2));
    R.rsk = R.rrn = R.rnm;
    if (qjl) {
        R.rsk = buffer_rsrc(a.packed + a.off_sketch + rec0 * (int64_t)(a.t.m / 8), (int)(a.n_tokens * (a.t.m / 8)));
        R.rrn = buffer_rsrc(a.packed + a.off_rnorm + rec0 * 2, (int)(a.n_tokens * 2));
    }
    return R;
}

// The binade-grid encode of one tensor (bf16 input, b <= 4, d <= 128; with the Gaussian sketch
// m <= 128): one 12-wave block per CU (three waves per SIMD), waves walking the block's tiles with
// the next tile's loads in flight.  Plain-KV skips the signs and the transform.
template <int D, int B, bool QJL>
__global__ __launch_bounds__(64 * kFqWaves, 1) void encode_fq_kernel(EncodeArgs a) {
    constexpr int NWV = kFqWaves, NTH = 64 * NWV;
    constexpr int C = D / 4, NKB = D / 32;
    static_assert(B <= 4 && D <= 128, "the binade grid serves b <= 4 at d <= 128");
    __shared__ __attribute__((aligned(16))) uint32_t fq_lds[fq_lds_bytes<D, B, QJL>() / 4];
    uint8_t* const ldsb = reinterpret_cast<uint8_t*>(fq_lds);
    const int64_t st = blockIdx.x / a.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int m = QJL ? a.t.m : 0;
    const bool rht = QJL && a.t.sketch == 1;
    const bool plain = a.t.rotation == 1;         // Plain-KV: no sign flip, no WHT
    const int tid = (int)threadIdx.x;
    fq_stage_tables<D, B, QJL>(ldsb, a.t, head, m, rht, 2 * NKB, tid);
    fq_stage_hadamard<D, B>(ldsb, 0, a.t.signs + (int64_t)head * D, false, tid, NTH);
    if (rht) fq_stage_hadamard<D, B>(ldsb, 2 * NKB, a.t.signs2 + (int64_t)head * D, true, tid, NTH);
    __syncthreads();

    const int lane = tid & 63;
    const int v = lane & 15, g = lane >> 4;
    const int wave = wave_id();
    const FqBufs R = fq_bufs<D, B>(a, st, QJL);
    uint32_t w[D / 8];
    const int64_t t_first = tb0 + wave;
    bload<2 * C, 16>(R.rx, (uint32_t)(t_first * 16 + v) * (2 * D) + 2 * g * C, 0u, w);
#pragma unroll 1
    for (int64_t t = t_first; t < tb1; t += NWV) {
        // keep the LDS operand tables in LDS (re-read per pass) instead of pinned in registers
        asm volatile("" ::: "memory");
        fq_encode_group<D, B, QJL>(ldsb, 0, 2 * NKB, rht, plain, m, R, w, t, t + NWV, tb1, a.n_tokens, lane);
    }
}

template <int D, int B, bool QJL>
__global__ __launch_bounds__(64 * kFqWaves, 1) void encode_kv_kernel(EncodeArgs ak, EncodeArgs av) {
    constexpr int NWV = kFqWaves, NTH = 64 * NWV;
    constexpr int C = D / 4, NKB = D / 32;
    static_assert(B <= 4 && D <= 128, "the binade grid serves b <= 4; the fused launch d <= 128");
    __shared__ __attribute__((aligned(16))) uint32_t fq_lds[fq_lds_bytes<D, B, QJL>() / 4];
    uint8_t* const ldsb = reinterpret_cast<uint8_t*>(fq_lds);

    const int64_t st = blockIdx.x / ak.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * ak.blocks_per_stream;
    const int64_t tb0 = sub * ak.tiles_per_block;
    const int64_t tb1 = tb0 + ak.tiles_per_block < ak.tiles_per_stream ? tb0 + ak.tiles_per_block : ak.tiles_per_stream;
    const int hk = (int)(st % ak.t.n_heads), hv = (int)(st % av.t.n_heads);
    const int m = QJL ? ak.t.m : 0;
    const bool rht = QJL && ak.t.sketch == 1;
    const int nS = !QJL ? 0 : (rht ? 2 * NKB : m * D / 512);     // window pieces of S / the RHT tiles
    const int pSk = 2 * NKB, pAv = 2 * NKB + nS;
    const int tid = (int)threadIdx.x;

    fq_stage_tables<D, B, QJL>(ldsb, ak.t, hk, m, rht, pSk, tid);
    fq_stage_hadamard<D, B>(ldsb, 0, ak.t.signs + (int64_t)hk * D, false, tid, NTH);
    if (rht) fq_stage_hadamard<D, B>(ldsb, pSk, ak.t.signs2 + (int64_t)hk * D, true, tid, NTH);
    fq_stage_hadamard<D, B>(ldsb, pAv, av.t.signs + (int64_t)hv * D, false, tid, NTH);
    __syncthreads();

    const int lane = tid & 63;
    const int v = lane & 15, g = lane >> 4;
    const int wave = wave_id();
    const FqBufs RK = fq_bufs<D, B>(ak, st, QJL), RV = fq_bufs<D, B>(av, st, false);
    uint32_t wk[D / 8], wv[D / 8];
    const int64_t t_first = tb0 + wave;
    bload<2 * C, 16>(RK.rx, (uint32_t)(t_first * 16 + v) * (2 * D) + 2 * g * C, 0u, wk);
    bload<2 * C, 16>(RV.rx, (uint32_t)(t_first * 16 + v) * (2 * D) + 2 * g * C, 0u, wv);
#pragma unroll 1
    for (int64_t t = t_first; t < tb1; t += NWV) {
        asm volatile("" ::: "memory");
        fq_encode_group<D, B, QJL>(ldsb, 0, pSk, rht, false, m, RK, wk, t, t + NWV, tb1, ak.n_tokens, lane);
        fq_encode_group<D, B, false>(ldsb, pAv, 0, false, false, 0, RV, wv, t, t + NWV, tb1, av.n_tokens, lane);
    }
}

// whether the fused key + value launch serves this pair (the binade grid for both, the same d,
// b and rotation with the WHT, one codebook, values without a sketch, the keys' tables within the
// window pieces)
template <int D, int B>
static bool fq_kv_fits(const EncodeArgs& ak, const EncodeArgs& av) {
    if (ak.t.fq_grid == nullptr || av.t.fq_grid == nullptr || ak.t.rotation != 0 || av.t.rotation != 0) return false;
    if (av.t.m != 0) return false;
    const int64_t lim = (int64_t)1 << 31;
    if (ak.n_tokens * 2 * D >= lim || ak.n_tokens * (D * B / 8) >= lim) return false;
    constexpr int nA = 2 * (D / 32);
    int nS = 0;
    if (ak.t.m > 0) {
        const bool rht = ak.t.sketch == 1;
        if (!rht && (ak.t.m > 128 || (ak.t.m * D) % 512 != 0)) return false;
        nS = rht ? nA : ak.t.m * D / 512;
    }
    return 2 * nA + nS <= FqLayout<B>::cap;
}

template <int D, int B>
static hipError_t launch_kv_db(const EncodeArgs& ak, const EncodeArgs& av, int num_cus, hipStream_t s, bool* fused) {
    *fused = false;
    if (!fq_kv_fits<D, B>(ak, av)) return hipSuccess;
    *fused = true;
    EncodeArgs k = ak, v = av;
    const bool qjl = ak.t.m > 0;
    const void* kern = qjl ? reinterpret_cast<const void*>(&encode_kv_kernel<D, B, true>)
                           : reinterpret_cast<const void*>(&encode_kv_kernel<D, B, false>);
    const int64_t target = (int64_t)num_cus * blocks_per_cu(kern, 0, 64 * kFqWaves);
    int64_t bps = (target + ak.n_streams - 1) / ak.n_streams;
    if (bps > ak.tiles_per_stream) bps = ak.tiles_per_stream;
    if (bps < 1) bps = 1;
    k.blocks_per_stream = v.blocks_per_stream = bps;
    k.tiles_per_block = v.tiles_per_block = (ak.tiles_per_stream + bps - 1) / bps;
    const dim3 grid((unsigned)(ak.n_streams * bps));
    if (qjl) hipLaunchKernelGGL((encode_kv_kernel<D, B, true>), grid, dim3(64 * kFqWaves), 0, s, k, v);
    else hipLaunchKernelGGL((encode_kv_kernel<D, B, false>), grid, dim3(64 * kFqWaves), 0, s, k, v);
    return hipGetLastError();
}

// keys and values of the same tokens in one launch where fq_kv_fits holds (*fused = true); else
// nothing is launched and *fused = false (the caller encodes the two tensors apart)
hipError_t launch_encode_kv(const EncodeArgs& ak, const EncodeArgs& av, int num_cus, hipStream_t s, bool* fused) {
    *fused = false;
    if (ak.t.d != av.t.d || ak.t.b != av.t.b || ak.n_streams != av.n_streams || ak.n_tokens != av.n_tokens) return hipSuccess;
    switch (ak.t.d * 16 + ak.t.b) {
        case 64 * 16 + 1: return launch_kv_db<64, 1>(ak, av, num_cus, s, fused);
        case 64 * 16 + 2: return launch_kv_db<64, 2>(ak, av, num_cus, s, fused);
        case 64 * 16 + 3: return launch_kv_db<64, 3>(ak, av, num_cus, s, fused);
        case 64 * 16 + 4: return launch_kv_db<64, 4>(ak, av, num_cus, s, fused);
        case 128 * 16 + 1: return launch_kv_db<128, 1>(ak, av, num_cus, s, fused);
        case 128 * 16 + 2: return launch_kv_db<128, 2>(ak, av, num_cus, s, fused);
        case 128 * 16 + 3: return launch_kv_db<128, 3>(ak, av, num_cus, s, fused);
        case 128 * 16 + 4: return launch_kv_db<128, 4>(ak, av, num_cus, s, fused);
    }
    return hipSuccess;
}

// binade-grid launch: bf16 input, b <= 4, the table built for this codebook, and the Hadamard
// tiles plus S (or the randomized Hadamard tiles) within the pieces of the centroid window; the
// Gaussian sketch also needs m <= 128 (one sketch word per lane part)
template <int D, int B, bool QJL>
static bool fq_fits(const EncodeArgs& a) {
    if (a.t.fq_grid == nullptr) return false;
    // the binade-grid kernel addresses one stream's input and record planes with 32-bit offsets
    const int64_t lim = (int64_t)1 << 31;
    if (a.n_tokens * 2 * D >= lim || a.n_tokens * (D * B / 8) >= lim) return false;
    if constexpr (QJL) {
        constexpr int nA = 2 * (D / 32);
        const bool rht = a.t.sketch == 1;
        if (!rht && (a.t.m > 128 || (a.t.m * D) % 512 != 0)) return false;
        const int nS = rht ? nA : a.t.m * D / 512;
        return nA + nS <= FqLayout<B>::cap;
    }
    return 2 * (D / 32) <= FqLayout<B>::cap;
}

template <int D, int B, bool QJL>
static hipError_t launch_fq(const EncodeArgs& a, int num_cus, hipStream_t s) {
    EncodeArgs b = a;
    b.grid_rep_log2 = 0;
    const void* kern = reinterpret_cast<const void*>(&encode_fq_kernel<D, B, QJL>);
    const int threads = 64 * kFqWaves;                                 // static LDS only
    const int64_t target = (int64_t)num_cus * blocks_per_cu(kern, 0, threads);
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    const dim3 grid((unsigned)(a.n_streams * bps));
    hipLaunchKernelGGL((encode_fq_kernel<D, B, QJL>), grid, dim3(threads), 0, s, b);
    return hipGetLastError();
}

template <int D, int B, bool QJL, bool BF16>
static hipError_t launch_one(const EncodeArgs& a, int num_cus, hipStream_t s) {
    // (at d = 256 the binade grid measured slower than the search grid without the sketch, and the
    // sketch spills at three waves per SIMD)
    if constexpr (BF16 && B <= 4 && D <= 128) {
        if (fq_fits<D, B, QJL>(a)) return launch_fq<D, B, QJL>(a, num_cus, s);
    }
    EncodeArgs b = a;
    const int L = 1 << B;
    // S lives in LDS whenever it fits beside the rest (160 KiB per CU; for d = 256 and m = 256 the
    // 128 KiB of S leave room for one block per CU); the grid is held in up to 16 copies (8 with the
    // sketch) within 16 KiB / 8 KiB, fewer if S needs the room
    constexpr size_t kLdsMax = 163840;
    const size_t grid_bytes = (size_t)(a.t.G + 3) * 8;
    const size_t fixed = (size_t)(L + 4) * 4 + (BF16 ? (size_t)2 * (D / 32) * 64 * 16 : 0);
    // the randomized Hadamard sketch of bf16 input keeps its ±1 tiles (the size of the A tiles) in
    // place of S
    const bool rht_tiles = QJL && BF16 && a.t.sketch == 1;
    const size_t s_bytes = rht_tiles ? (size_t)2 * (D / 32) * 64 * 16 : (size_t)a.t.m * D * 2;
    const bool s_lds = QJL && (D <= 128 || fixed + grid_bytes + s_bytes <= kLdsMax);   // always for d <= 128
    int rl = QJL ? 3 : 4;
    while (rl > 0 && ((grid_bytes << rl) > (QJL ? 8192u : 16384u) ||
                      (s_lds && fixed + (grid_bytes << rl) + s_bytes > kLdsMax)))
        --rl;
    b.grid_rep_log2 = rl;
    const size_t head_bytes = (grid_bytes << rl) + fixed;
    const size_t lds = head_bytes + (s_lds ? s_bytes : 0);
    const void* kern = s_lds ? reinterpret_cast<const void*>(&encode_kernel<D, B, QJL, BF16, true>)
                             : reinterpret_cast<const void*>(&encode_kernel<D, B, QJL, BF16, (D <= 128)>);
    if (lds > 65536) {           // above the default dynamic LDS limit: raise it once per kernel
        static std::mutex mu;
        static bool raised = false;
        std::lock_guard<std::mutex> lock(mu);
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
            if (e != hipSuccess) return e;
            raised = true;
        }
    }
    // one wave of blocks: as many blocks as fit on every CU at once
    const int threads = 64 * (s_lds ? enc_waves<D, QJL, BF16, true>() : enc_waves<D, QJL, BF16, (D <= 128)>());
    const int64_t target = (int64_t)num_cus * blocks_per_cu(kern, lds, threads);
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    const dim3 grid((unsigned)(a.n_streams * bps));
    if constexpr (D <= 128) {
        hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, true>), grid, dim3(threads), lds, s, b);
    } else {
        if (s_lds) hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, true>), grid, dim3(threads), lds, s, b);
        else hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, false>), grid, dim3(threads), lds, s, b);
    }
    return hipGetLastError();
}

template <int D, int B>
static hipError_t launch_db(const EncodeArgs& a, bool bf16, int num_cus, hipStream_t s) {
    const bool qjl = a.t.m > 0;
    if (bf16) return qjl ? launch_one<D, B, true, true>(a, num_cus, s) : launch_one<D, B, false, true>(a, num_cus, s);
    return qjl ? launch_one<D, B, true, false>(a, num_cus, s) : launch_one<D, B, false, false>(a, num_cus, s);
}

template <int D>
static hipError_t launch_d(const EncodeArgs& a, bool bf16, int num_cus, hipStream_t s) {
    switch (a.t.b) {
        case 1: return launch_db<D, 1>(a, bf16, num_cus, s);
        case 2: return launch_db<D, 2>(a, bf16, num_cus, s);
        case 3: return launch_db<D, 3>(a, bf16, num_cus, s);
        case 4: return launch_db<D, 4>(a, bf16, num_cus, s);
        case 5: return launch_db<D, 5>(a, bf16, num_cus, s);
        case 6: return launch_db<D, 6>(a, bf16, num_cus, s);
        case 7: return launch_db<D, 7>(a, bf16, num_cus, s);
        case 8: return launch_db<D, 8>(a, bf16, num_cus, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_encode(const EncodeArgs& a, bool x_bf16, int num_cus, hipStream_t s) {
    switch (a.t.d) {
        case 64: return launch_d<64>(a, x_bf16, num_cus, s);
        case 128: return launch_d<128>(a, x_bf16, num_cus, s);
        case 256: return launch_d<256>(a, x_bf16, num_cus, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
