// Encode kernel ("Ablation, Statistical Inference, and Validation for KV-Cache Compression",
// §2 TurboQuant): per vector x, n = ||x||, y = H (x ⊙ s) / (sqrt(d) n), idx_j = #{i : t_i <= y_j},
// b-bit packing; with m > 0 also e = y - c[idx], ||e|| and sign(S e) (1-bit QJL of the residual).
//
// Work split: one wave64 = 16 vectors x 4 parts (see common.hpp).  Waves walk a contiguous range of
// 16-vector tiles, so the per-head sign constants are reloaded only when the stream changes.
// Search: a uniform grid over y in [-1,1] held in LDS maps y to the one threshold that can lie in
// its cell plus the count of thresholds below; one compare finishes the search for any b.
// S·e: v_mfma_f32_16x16x32_f16 with the lane's own residual as the B operand (lane l = vector
// l%16, k-block l/16 matches the MFMA operand layout): 2^14 e rounded to the nearest fp16
// (|2^14 e| < 2^15 always, so only precision is lost), the precision the sign decisions are
// defined in; S stored as fp16 values; exact products, accumulation in fp32.
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace tq {

template <int D, int B, bool QJL, bool BF16, bool S_LDS>
__global__ __launch_bounds__(256, ((D > 128 && (QJL || !BF16)) || (QJL && !BF16) ? 1 : (D > 128 ? 2 : 3))) void encode_kernel(EncodeArgs a) {
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
    for (int i = threadIdx.x; i < ((G + 3) << rl); i += blockDim.x) {
        const int c = i >> rl;
        lds[2 * i] = a.t.grid[2 * c];
        lds[2 * i + 1] = a.t.grid[2 * c + 1];
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
    const int wave = threadIdx.x >> 6;
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
    for (int64_t t = tb0 + wave * NG; t < tb1; t += 4 * NG) {
        // keep the LDS operand tables in LDS (re-read per pass) instead of pinned in registers
        asm volatile("" ::: "memory");
        half8 bh[NG][QJL ? C / 8 : 1];
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
                            const floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, lds_A[(h * NKB + kb) * 64 + lane]), Bv,
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
                if (t + 4 * NG < tb1) load_group(nxt[gi], t + 4 * NG + gi);
                if (!plain) fwht_slots<C, 8>(x);
            } else {
#pragma unroll
                for (int s = 0; s < C; ++s) {
                    const float xv = u2f(w[s]);
                    n2 = fmaf(xv, xv, n2);
                    x[s] = plain ? xv : xv * sg[s];
                }
                if (t + 4 * NG < tb1) load_group(nxt[gi], t + 4 * NG + gi);
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
                // B operands: lane's residual slots [8k, 8k+8) for k-step k, in fp16 (nearest even)
#pragma unroll
                for (int k = 0; k < C / 8; ++k) {
                    u32x4 hv;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        hv[u] = __builtin_bit_cast(uint32_t, half2v{(_Float16)x[8 * k + 2 * u], (_Float16)x[8 * k + 2 * u + 1]});
                    bh[gi][k] = __builtin_bit_cast(half8, hv);
                }
            }
        }

        if constexpr (QJL && BF16) {
          if (a.t.sketch == 1) {
            // randomized Hadamard sketch z = H (e ⊙ s2) (m = d): the rotation's 32-point block on
            // fp16 MFMA with the s2 tiles as A and the residual's fp16 values as B, then
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
                        const floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[gi][kb], floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
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
                if (validv[gi] && g == 0)
                    *reinterpret_cast<_Float16*>(a.packed + a.off_rnorm + vecv[gi] * 2) =
                        (_Float16)(sqrtf(e2) * (1.0f / 16384.0f));
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
            auto sketch_word = [&](int wb, int nt, auto full) {
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
                                const half8 A = *reinterpret_cast<const half8*>(
                                    S_LDS ? Sg + (tau * KS + k) * 512 : Sg + 4 * tau * D + 8 * k);
#pragma unroll
                                for (int gi = 0; gi < NG; ++gi)
                                    acc[gi][tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[gi][k], acc[gi][tl], 0, 0, 0);
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
                    // issue order: the first kPD S reads, then per step its MFMA and the read kPD
                    // steps ahead, so each read has kPD steps of matrix work to land
                    constexpr int kPD = 4;
                    __builtin_amdgcn_sched_group_barrier(0x100, kPD, 0);
#pragma unroll
                    for (int p = 0; p < 8 * KS; ++p) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
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
                if (validv[gi] && g == 0)
                    *reinterpret_cast<_Float16*>(a.packed + a.off_rnorm + vecv[gi] * 2) =
                        (_Float16)(sqrtf(e2) * (1.0f / 16384.0f));
            }
        }
    }
}

// resident blocks per CU of kernel k at `lds` bytes of dynamic LDS (cached per kernel and size)
static int blocks_per_cu(const void* k, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<const void*, size_t>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({k, lds});
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 256, lds) != hipSuccess || n < 1) n = 1;
    cache[{k, lds}] = n;
    return n;
}

template <int D, int B, bool QJL, bool BF16>
static hipError_t launch_one(const EncodeArgs& a, int num_cus, hipStream_t s) {
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
    // one wave of blocks: as many 256-thread blocks as fit on every CU at once
    const int64_t target = (int64_t)num_cus * blocks_per_cu(kern, lds);
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    const dim3 grid((unsigned)(a.n_streams * bps));
    if constexpr (D <= 128) {
        hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, true>), grid, dim3(256), lds, s, b);
    } else {
        if (s_lds) hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, true>), grid, dim3(256), lds, s, b);
        else hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, false>), grid, dim3(256), lds, s, b);
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
