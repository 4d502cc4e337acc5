// Fused GQA decode attention over the packed cache ("Ablation, Statistical Inference, and
// Validation for KV-Cache Compression", eq. (1) T = softmax(QK^T/sqrt(d))V, with the scores
// estimated on compressed keys as in §2 TurboQuant / SpectralQuant paragraphs).
//
// Split-K (flash-decoding): one wave per (stream = batch·n_kv + kv head, token split).  Per chunk
// of 32 tokens:
//   scores  D[token][q] = K̂ Q^T on v_mfma_f32_16x16x32_f16 (A = dequantised keys, lane = token
//           l%16 with its packed k-block l/16; B = the rotated queries as fp16 hi + lo parts, two
//           products), plus the QJL term <p, 2σ-1> with A = ±1 sketch bits and B = fp16 S·q_rot;
//   softmax online in base 2; the score accumulator of lane (q = l%16, g = l/16) holds tokens
//           {4g+i, 16+4g+i}, exactly the k-block g of the B operand of the next product;
//   values  O^T[coord][q] += V̂^T W^T (A = dequantised values, lane = coordinate row l%16 over its
//           8 tokens), accumulated in the rotated domain — no per-token inverse transform.
// A combine kernel merges the splits and applies the inverse rotation s_V ⊙ H(·)/sqrt(d) once.
#include "common.hpp"
#include "kernels.hpp"

namespace tq {

// plain v_max_f32: the operands come out of lane swaps, which the compiler cannot prove quiet, so
// fmaxf would first canonicalise both (the logits are never signalling NaNs)
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float max4(float t) {
    float a = t, b = t;
    xswap16(a, b);
    t = vmax(a, b);
    a = t;
    b = t;
    xswap32(a, b);
    return vmax(a, b);
}

// Everything one 32-token chunk needs, loaded with wide per-lane loads.  Lane (l16, g):
//   kw[T]  packed K chunk g of token 16T + l16 (score A operand rows)
//   ks[T]  its sketch bytes [g·m/32, (g+1)·m/32)
//   kn/kr/vn[T]  the 4 fp16 norms of tokens 16T + 4g + {0..3} (the rows its score outputs hold)
//   vw[r]  packed V bytes of coordinates [NT·l16, NT·l16 + NT) of token τ(g, r), where
//          τ(g, r) = 4g + r for r < 4 and 16 + 4g + (r - 4) otherwise
template <int NWK, int NWV, int NKS>
struct AttnChunk {
    uint32_t kw[2][NWK];
    uint32_t ks[2][NKS + 1];     // covering aligned dwords; the lane's bytes start at byte (g m/32) % 4
    u32x2 kn[2], kr[2], vn[2];
    uint32_t vw[8][NWV];
};

template <int D, int BK, int BV>
struct AttnGeom {
    static constexpr int C = D / 4, KS = C / 8;
    static constexpr int PK = lut_group_c(BK), NEK = 1 << (PK * BK);
    static constexpr int NWK = (C * BK + 31) / 32, CBK = C * BK / 8, CAK = cmin(pow2_align(CBK), 16);
    static constexpr int NT = D / 16, VB = NT * BV / 8, VA = cmin(pow2_align(VB), 16);
    static constexpr int NWV = (NT * BV + 31) / 32;
    static constexpr int KROW = D * BK / 8, VROW = D * BV / 8;
    static constexpr bool VPAIR = BV == 4;           // two-token pair LUT for 4-bit values
    static constexpr int NKS = D >= 256 ? 2 : 1;     // sketch words per lane (m <= d)
    // The K dequantisation LUT and the value pair LUT are read at random entries.  LDS has 32
    // banks of 4 bytes and serves 128 bytes per cycle, i.e. 128/E lanes of an E-byte read at once;
    // holding 128/E copies with entry e of copy c at (e·copies + c)·E gives every lane of such a
    // phase its own banks (lane l reads copy l % copies).  Done when the copies fit in 32 KiB.
    // A K entry holds the fp16 hi parts of 2^12 c for its PK coordinates, then their lo parts.
    static constexpr int KE = 4 * PK;                // bytes per K LUT entry
    static constexpr int KR = (NEK * KE * (128 / KE) <= 32768) ? 128 / KE : 1;
    static constexpr int VR = VPAIR ? 32 : 1;        // copies of the 1 KiB value pair LUT
    // 4-bit keys and values: the LUTs have 256 entries of 4 bytes each (V pair; K hi pair; K lo
    // pair), so two tables of 256-byte rows hold 32 copies of each: row e of the first is
    // [V pair x 32 | K hi pair x 32], row e of the second (64 KiB on) [K lo pair x 32 | unused].  A
    // lane's address is the byte index shifted by 8 or-ed with its copy offset: one v_perm_b32 per
    // lookup, and the lo pair is the same address plus a constant (the read's immediate offset).
    // Every read is 4 bytes into the register the MFMA operand needs, and lanes l, l + 16 of a
    // 32-lane phase use different banks.
    static constexpr bool KV256 = VPAIR && PK == 2 && NEK == 256;
    static constexpr int KV_LO = 65536 - 128;        // lo pair address - hi pair address
    // threads per block: the 128 KiB of tables are shared by the waves of one block per CU (see
    // attn_threads)
    static constexpr int THREADS = (KV256 && D <= 128) ? 512 : 256;
};

// a * b + c with a the fp16 number i of the four in v (the compiler folds the widening into the
// fma: v_fma_mix_f32)
__device__ __forceinline__ float fma_h(const u32x2& v, int i, float b, float c) {
    const uint32_t w = v[i >> 1];
    const _Float16 a = __builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
    return fmaf((float)a, b, c);
}

// byte offset (idx << 8) | off, idx = byte `which` of w, off < 256: D = {0, 0, w.byte[which], off.byte0}
__device__ __forceinline__ uint32_t row256(uint32_t w, uint32_t off, int which) {
    return __builtin_amdgcn_perm(w, off, 0x0c0c0000u | ((uint32_t)(4 + which) << 8));
}

// Buffer resources of one stream's planes and the lane's loop-invariant byte offsets within a
// chunk (full chunks; the chunk's first token enters as the wave-uniform scalar offset)
struct AttnRes {
    __amdgpu_buffer_rsrc_t kidx, ksk, kn, kr, vidx, vn;
    uint32_t o_kw, o_ks, o_n, o_vw;
};

// Per-wave base pointers of one stream (chunk offsets are added as wave-uniform values).
struct AttnPtrs {
    const uint8_t* kidx;
    const uint8_t* ksk;
    const uint8_t* kn;
    const uint8_t* kr;
    const uint8_t* vidx;
    const uint8_t* vn;
};

template <int D, int BK, int BV, bool QJL>
__device__ __forceinline__ void attn_load_full(AttnChunk<AttnGeom<D, BK, BV>::NWK, AttnGeom<D, BK, BV>::NWV, AttnGeom<D, BK, BV>::NKS>& c,
                                               const AttnRes& R, int64_t t0, int m) {
    using Gm = AttnGeom<D, BK, BV>;
    const uint32_t tk = (uint32_t)t0;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        bload<Gm::CBK, Gm::CAK>(R.kidx, R.o_kw, (tk + 16 * T) * Gm::KROW, c.kw[T]);
        if constexpr (QJL) {
            // the covering aligned dwords of the lane's m/32 sketch bytes (see attn_load)
            const uint32_t so = (tk + 16 * T) * (uint32_t)(m / 8);
#pragma unroll
            for (int k = 0; k <= Gm::NKS; ++k) c.ks[T][k] = __builtin_amdgcn_raw_buffer_load_b32(R.ksk, R.o_ks + 4 * k, so, 0);
        }
        const uint32_t sn = 2 * tk + 32 * T;
        c.kn[T] = __builtin_amdgcn_raw_buffer_load_b64(R.kn, R.o_n, sn, 0);
        if constexpr (QJL) c.kr[T] = __builtin_amdgcn_raw_buffer_load_b64(R.kr, R.o_n, sn, 0);
        c.vn[T] = __builtin_amdgcn_raw_buffer_load_b64(R.vn, R.o_n, sn, 0);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int tr = r < 4 ? r : 16 + (r - 4);          // τ(g, r) - 4g
        bload<Gm::VB, Gm::VA>(R.vidx, R.o_vw, (tk + tr) * Gm::VROW, c.vw[r]);
    }
}

template <int D, int BK, int BV, bool QJL, bool FULL>
__device__ __forceinline__ void attn_load(AttnChunk<AttnGeom<D, BK, BV>::NWK, AttnGeom<D, BK, BV>::NWV, AttnGeom<D, BK, BV>::NKS>& c,
                                          const AttnPtrs& P, int64_t t0, int64_t t_end, int l16, int g, int m) {
    using Gm = AttnGeom<D, BK, BV>;
    // wave-uniform chunk bases, 32-bit lane offsets
    const uint8_t* kb = P.kidx + t0 * Gm::KROW;
    const uint8_t* vb = P.vidx + t0 * Gm::VROW;
    const uint32_t koff = l16 * Gm::KROW + g * Gm::CBK;
    const uint32_t voff = (4 * g) * Gm::VROW + l16 * Gm::VB;
    const uint32_t noff = 8 * g;                       // 4 fp16 norms of tokens 4g..4g+3
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        const int rem = (int)(t_end - t0);             // tokens left (FULL: >= 32)
        if (FULL || 16 * T + l16 < rem) {
            load_bytes<Gm::CBK, Gm::CAK>(kb + koff + T * 16 * Gm::KROW, c.kw[T]);
            if constexpr (QJL) {
                // the lane's m/32 sketch bytes start at any byte offset: read the covering aligned
                // dwords and funnel-shift (branch-free, so the load counters stay static).  Bytes past
                // m/32 are never used; the over-read stays inside the packed buffer, whose norm
                // planes follow the sketch plane.
                // (the byte offset within the dword is (g m/32) % 4: rows are multiples of 4 bytes)
                const uint8_t* sp = P.ksk + (t0 + 16 * T + l16) * (m / 8) + ((g * (m / 32)) & ~3);
#pragma unroll
                for (int k = 0; k <= Gm::NKS; ++k) c.ks[T][k] = reinterpret_cast<const uint32_t*>(sp)[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < Gm::NWK; ++k) c.kw[T][k] = 0u;
#pragma unroll
            for (int k = 0; k <= Gm::NKS; ++k) c.ks[T][k] = 0u;
        }
        if (FULL || 16 * T + 4 * g + 4 <= rem) {
            c.kn[T] = *reinterpret_cast<const u32x2*>(P.kn + t0 * 2 + noff + 32 * T);
            if constexpr (QJL) c.kr[T] = *reinterpret_cast<const u32x2*>(P.kr + t0 * 2 + noff + 32 * T);
            c.vn[T] = *reinterpret_cast<const u32x2*>(P.vn + t0 * 2 + noff + 32 * T);
        } else {
            uint32_t e0[4] = {0, 0, 0, 0}, e1[4] = {0, 0, 0, 0}, e2[4] = {0, 0, 0, 0};
            for (int i = 0; i < 4; ++i)
                if (16 * T + 4 * g + i < rem) {
                    const int64_t o = t0 * 2 + noff + 32 * T + 2 * i;
                    e0[i] = *reinterpret_cast<const uint16_t*>(P.kn + o);
                    if constexpr (QJL) e1[i] = *reinterpret_cast<const uint16_t*>(P.kr + o);
                    e2[i] = *reinterpret_cast<const uint16_t*>(P.vn + o);
                }
            c.kn[T] = u32x2{e0[0] | (e0[1] << 16), e0[2] | (e0[3] << 16)};
            c.kr[T] = u32x2{e1[0] | (e1[1] << 16), e1[2] | (e1[3] << 16)};
            c.vn[T] = u32x2{e2[0] | (e2[1] << 16), e2[2] | (e2[3] << 16)};
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int tr = r < 4 ? r : 16 + (r - 4);          // τ(g, r) - 4g
        if (FULL || 4 * g + tr < (int)(t_end - t0)) load_bytes<Gm::VB, Gm::VA>(vb + voff + tr * Gm::VROW, c.vw[r]);
        else {
#pragma unroll
            for (int k = 0; k < Gm::NWV; ++k) c.vw[r][k] = 0u;
        }
    }
}

__device__ __forceinline__ float half_of(const u32x2& v, int i) {
    const uint32_t w = v[i >> 1];
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
}

// running state of the online softmax for the wave's 16 query columns
template <int NT>
struct AttnState {
    floatx4 oacc[NT];
    float m_run, l_run;
};

template <int D, int BK, int BV, bool QJL, bool FULL, bool PQ>
__device__ __forceinline__ void attn_chunk(const AttnChunk<AttnGeom<D, BK, BV>::NWK, AttnGeom<D, BK, BV>::NWV, AttnGeom<D, BK, BV>::NKS>& cur,
                                           AttnState<AttnGeom<D, BK, BV>::NT>& S, int64_t t0, int64_t t_end,
                                           int g, int mks,
                                           const half8 (&qb)[AttnGeom<D, BK, BV>::KS],
                                           const half8 (&qbl)[AttnGeom<D, BK, BV>::KS], const half8* pb, float rowf,
                                           const uint8_t* kl, const _Float16* vlut, const uint8_t* vl2,
                                           const uint8_t* sg8, const uint8_t* kvl, uint32_t koff, uint32_t voff,
                                           uint32_t ksh) {
    using Gm = AttnGeom<D, BK, BV>;
    constexpr int KS = Gm::KS, PK = Gm::PK, NT = Gm::NT;
    // ---- scores for the two 16-token tiles ----------------------------------------------------
    // K̂ Qᵀ as hi·hi + lo·hi + hi·lo of the fp16 parts of 2^12 c and of the queries: only the fp32
    // accumulation rounds, so the logits stay fp32-accurate however sharp the softmax.
    float lg[8];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        floatx4 s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            constexpr int KST = Gm::KR * Gm::KE;      // bytes between entries of one copy
            half8 ka, kal;
            if constexpr (PK == 4) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t f = get_bits<4 * BK>(cur.kw[T], (8 * k + 4 * h) * BK);
                    const half8 e = *reinterpret_cast<const half8*>(kl + f * KST);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        ka[4 * h + u] = e[u];
                        kal[4 * h + u] = e[4 + u];
                    }
                }
            } else if constexpr (Gm::KV256) {
                // coordinates (8k + 2h, +1) are byte h of packed word k
                u32x4 kh, kq;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint8_t* e = kvl + row256(cur.kw[T][k], koff, h);
                    kh[h] = *reinterpret_cast<const uint32_t*>(e);
                    kq[h] = *reinterpret_cast<const uint32_t*>(e + Gm::KV_LO);
                }
                ka = __builtin_bit_cast(half8, kh);
                kal = __builtin_bit_cast(half8, kq);
            } else {
                static_assert(PK == 2, "attention keys use 2 or 4 coordinates per LUT entry");
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t f = get_bits<2 * BK>(cur.kw[T], (8 * k + 2 * h) * BK);
                    const half4 e = *reinterpret_cast<const half4*>(kl + f * KST);
                    ka[2 * h] = e[0];
                    ka[2 * h + 1] = e[1];
                    kal[2 * h] = e[2];
                    kal[2 * h + 1] = e[3];
                }
            }
            if constexpr (PQ) {
                // columns 0-7: query hi parts, 8-15: their lo parts; both key parts multiply both,
                // so columns 8-15 also carry lo·lo (2^-22 relative: below the fp32 accumulation)
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[k], s1, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kal, qb[k], s1, 0, 0, 0);
            } else {
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[k], s1, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kal, qb[k], s1, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qbl[k], s1, 0, 0, 0);
            }
        }
        if constexpr (PQ) {
            // column q + 8 holds hi·lo of query q: add it in (DPP row_shl:8 within each 16-lane row)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s1[i] += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(s1[i]), 0x108, 0xf, 0xf, true));
        }
        floatx4 s2 = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (QJL) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                // branch-free: steps past the sketch (k >= m/32) multiply a zero query operand
                const uint32_t wsk = __builtin_amdgcn_alignbit(cur.ks[T][(k >> 2) + 1], cur.ks[T][k >> 2], ksh);
                // the ±2^12 operand of the step's 8 sketch bits: one 16-byte entry per byte value
                const uint32_t sb = __builtin_amdgcn_ubfe(wsk, 8 * (k & 3), 8);
                const half8 sa = *reinterpret_cast<const half8*>(sg8 + sb * 64u);
                s2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, pb[k], s2, 0, 0, 0);
                if constexpr (!PQ) s2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, pb[KS + k], s2, 0, 0, 0);
            }
            if constexpr (PQ) {
                // column q + 8 holds the signs against the lo part of query q's projection
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s2[i] += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(s2[i]), 0x108, 0xf, 0xf, true));
            }
        }
        // output lane (q = l16, g) holds tokens t0 + 16T + 4g + i; the queries (and their sketch
        // projections) already carry the softmax scale in log2 units (and sqrt(pi/2)/m) and the
        // row's power of two, the keys 2^12 and the sign operand ±2^12, so the base-2 logit is
        // rowf · n16 · (s1 + r16 s2), with rowf the row factor (times 2^-12); lg holds
        // n16 (s1 + r16 s2) and rowf (> 0, the lane's own) is applied in the softmax
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sc = s1[i];
            if constexpr (QJL) sc = fma_h(cur.kr[T], i, s2[i], sc);
            float v = fma_h(cur.kn[T], i, sc, 0.0f);
            if (!FULL && t0 + 16 * T + 4 * g + i >= t_end) v = -INFINITY;
            lg[4 * T + i] = v;
        }
    }
    // ---- online softmax (base 2) per query column; rescale only when a running max moved ---------
    float cmax = lg[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, lg[r]);
    cmax = max4(cmax) * rowf;
    const float m_new = fmaxf(S.m_run, cmax);
    if (__builtin_amdgcn_read_exec() & __ballot(m_new != S.m_run)) {
        const float alpha = __builtin_amdgcn_exp2f(S.m_run - m_new);
        S.l_run *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) S.oacc[n] *= alpha;
        S.m_run = m_new;
    }
    float wsum = 0.0f;
    half8 wb;
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // tokens r, r + 1 of the lane's eight: fp16 norms h of the pair word of tile T
            const int r = 4 * T + 2 * h;
            const half2v wh = {(_Float16)__builtin_amdgcn_exp2f(fmaf(rowf, lg[r], -m_new)),
                               (_Float16)__builtin_amdgcn_exp2f(fmaf(rowf, lg[r + 1], -m_new))};
            wsum = __builtin_amdgcn_fdot2(wh, half2v{(_Float16)1.0f, (_Float16)1.0f}, wsum, false);
            const half2v wv = wh * __builtin_bit_cast(half2v, h ? cur.vn[T].y : cur.vn[T].x);
            wb[r] = wv[0];
            wb[r + 1] = wv[1];
        }
    S.l_run += wsum;
    // ---- values: A = V̂^T tile n (row = coordinate NT*l16 + n), 8 tokens of k-block g -------------
    if constexpr (Gm::VPAIR) {
        // tokens (2p, 2p+1) share one lookup: byte k of z[p][0] / z[p][1] = the two 4-bit indices of
        // tile 2k / 2k+1 of word j (tiles 8j..8j+7)
#pragma unroll
        for (int j = 0; j < Gm::NWV; ++j) {
            uint32_t ze[4], zo[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t w0 = cur.vw[2 * p][j], w1 = cur.vw[2 * p + 1][j];
                // one shift and one bit-field insert each (v_bfi_b32)
                ze[p] = ((w0 & 0x0f0f0f0fu) | ((w1 << 4) & ~0x0f0f0f0fu));
                zo[p] = ((w0 >> 4) & 0x0f0f0f0fu) | (w1 & ~0x0f0f0f0fu);
            }
#pragma unroll
            for (int q = 0; q < 8 && 8 * j + q < NT; ++q) {
                half8 va;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t z = (q & 1) ? zo[p] : ze[p];
                    uint32_t e;
                    if constexpr (Gm::KV256) e = *reinterpret_cast<const uint32_t*>(kvl + row256(z, voff, q >> 1));
                    else e = *reinterpret_cast<const uint32_t*>(vl2 + ((z >> (8 * (q >> 1))) & 0xffu) * (4 * Gm::VR));
                    const half2v hv = __builtin_bit_cast(half2v, e);
                    va[2 * p] = hv[0];
                    va[2 * p + 1] = hv[1];
                }
                S.oacc[8 * j + q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, wb, S.oacc[8 * j + q], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            half8 va;
#pragma unroll
            for (int r = 0; r < 8; ++r) va[r] = vlut[get_bits<BV>(cur.vw[r], n * BV)];
            S.oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, wb, S.oacc[n], 0, 0, 0);
        }
    }
}

// threads per block: with the shared 4-bit tables at d <= 128, three waves per SIMD when the
// query operand packs hi and lo parts (group <= 8: 163 VGPRs), else two
template <int D, int BK, int BV, bool PQ>
constexpr int attn_threads() { return AttnGeom<D, BK, BV>::THREADS == 512 && PQ ? 768 : AttnGeom<D, BK, BV>::THREADS; }

// PQ: at most 8 query heads per kv head, so the query operand carries hi parts in columns 0-7
// and lo parts in columns 8-15, and the scores take two products per step instead of three
template <int D, int BK, int BV, bool QJL, bool PQ>
__global__ __launch_bounds__((attn_threads<D, BK, BV, PQ>()), (attn_threads<D, BK, BV, PQ>() == 768 ? 3 : (D <= 128 ? 2 : 1)))
void attn_kernel(AttnArgs a) {
    using Gm = AttnGeom<D, BK, BV>;
    constexpr int C = Gm::C, KS = Gm::KS, PK = Gm::PK, NEK = Gm::NEK, NT = Gm::NT;
    constexpr int LV = 1 << BV;

    constexpr int KR = Gm::KR, KE = Gm::KE, VR = Gm::VR;
    constexpr bool KV = Gm::KV256;
    __shared__ uint32_t klut[KV ? 1 : NEK * KE / 4 * KR];          // copy c of entry e at (e KR + c) KE bytes
    __shared__ _Float16 vlut[LV];
    __shared__ uint32_t vlut2[Gm::VPAIR && !KV ? 256 * VR : 1];  // copy c of entry e at word e VR + c
    __shared__ uint32_t kvlut[KV ? 2 * 256 * 64 : 1];             // the two tables of 256-byte rows
    __shared__ u32x4 sgn8[QJL ? 256 * 4 : 1];                      // copy c of byte e's ±2^12 halves at e·4 + c
    // The query prep of the block's stream, when every wave of the block works on that one stream
    // (a.fused_q, chosen by the host): the query prep kernel's steps for the group's rows, in the same
    // order and precision, with the rows' operands left in LDS (q_rot and S q_rot in fp32, then per
    // row the fp16 hi and lo parts of 2^e q_rot q_scale and of 2^e S q_rot p_scale, and the row factor
    // 2^-e).  Thread i < m fetches row i of S first; wave r < group rotates row r.  The hi and lo
    // parts of row r's projection overwrite its fp32 values in place (halves r·256 + i and r·256 +
    // 128 + i), which only wave r reads, and before it writes.
    constexpr bool FQP = KV && PQ && D <= 128;
    constexpr int FQM = QJL ? 128 : 0;                             // m <= 128 on this path
    constexpr int FQS = 2 * D;                                     // halves per row of fq_h
    __shared__ float fq_rot[FQP ? 8 * D : 1];
    __shared__ __attribute__((aligned(16))) float fq_p[FQP && QJL ? 8 * 128 : 4];
    __shared__ __attribute__((aligned(16))) _Float16 fq_h[FQP ? 8 * FQS : 8];
    _Float16* const fq_ph = reinterpret_cast<_Float16*>(fq_p);
    __shared__ float fq_rf[FQP ? 8 : 1];
    u32x4 srow[FQP && QJL ? D / 8 : 1];
    if constexpr (FQP) {
        if (a.fused_q) {
            constexpr int PL = D / 64;
            const int wv = wave_id(), lane = threadIdx.x & 63;
            const int64_t st_b = ((int64_t)blockIdx.x * (blockDim.x >> 6)) / a.n_split;
            const int b_b = (int)(st_b / a.n_kv_heads), h_b = (int)(st_b - (int64_t)b_b * a.n_kv_heads);
            const int hs = (int)(st_b % a.tk.n_heads);
            if constexpr (QJL) {
                if ((int)threadIdx.x < a.tk.m) {
                    const u32x4* sp = reinterpret_cast<const u32x4*>(a.tk.S + ((int64_t)hs * a.tk.m + threadIdx.x) * D);
#pragma unroll
                    for (int k = 0; k < D / 8; ++k) srow[k] = sp[k];
                }
            }
            if (wv < a.group) {
                // lane l holds coordinates PL l + c: the low index bits in the lane, the rest as
                // lane-xor butterflies, stage by stage from the lowest bit
                const int64_t row = (int64_t)b_b * a.n_q_heads + (int64_t)h_b * a.group + wv;
                const bool rot = a.tk.rotation != 1;
                float v[PL];
                const float* sg = a.tk.signs + (int64_t)hs * D + PL * lane;
#pragma unroll
                for (int c = 0; c < PL; ++c) {
                    const int64_t j = row * D + PL * lane + c;
                    const float x = a.q_bf16 ? u2f(uint32_t(reinterpret_cast<const uint16_t*>(a.q)[j]) << 16)
                                             : reinterpret_cast<const float*>(a.q)[j];
                    v[c] = rot ? x * sg[c] : x;
                }
                if (rot) {
#pragma unroll
                    for (int h = 1; h < PL; h <<= 1)
#pragma unroll
                        for (int c = 0; c < PL; ++c)
                            if (!(c & h)) {
                                const float x0 = v[c], x1 = v[c + h];
                                v[c] = x0 + x1;
                                v[c + h] = x0 - x1;
                            }
#pragma unroll
                    for (int hl = 1; hl < 64; hl <<= 1) {
                        const bool hi = (lane & hl) != 0;
#pragma unroll
                        for (int c = 0; c < PL; ++c) {
                            const float o = __shfl_xor(v[c], hl);
                            v[c] = hi ? o - v[c] : v[c] + o;
                        }
                    }
                    const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
                    for (int c = 0; c < PL; ++c) v[c] *= inv;
                }
#pragma unroll
                for (int c = 0; c < PL; ++c) fq_rot[wv * D + PL * lane + c] = v[c];
            }
        }
    }
    if constexpr (KV) {
        // a straight copy of the prebuilt images in 16-byte pieces: a piece of table 0 in words
        // 0-31 of its row (piece index % 16 < 8) holds value pairs, all else comes from the K codec
        const u32x4* kimg = reinterpret_cast<const u32x4*>(a.tk.attn_img);
        const u32x4* vimg = reinterpret_cast<const u32x4*>(a.tv.attn_img);
        u32x4* dst = reinterpret_cast<u32x4*>(kvlut);
        // four pieces per round trip (8192 pieces)
        const int nt = (int)blockDim.x;
        for (int i = threadIdx.x; i < 2 * 256 * 64 / 4; i += 4 * nt) {
            u32x4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = i + u * nt;
                if (k < 2 * 256 * 64 / 4) w[u] = ((k >> 12) == 0 && (k & 15) < 8 ? vimg : kimg)[k];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = i + u * nt;
                if (k < 2 * 256 * 64 / 4) dst[k] = w[u];
            }
        }
    } else {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(a.tk.lut_hl);
        uint16_t* dst = reinterpret_cast<uint16_t*>(klut);
        for (int i = threadIdx.x; i < NEK * KR; i += blockDim.x) {
            const int e = i / KR, c = i - e * KR;
#pragma unroll
            for (int h = 0; h < 2 * PK; ++h) dst[(e * KR + c) * 2 * PK + h] = src[e * 2 * PK + h];
        }
    }
    for (int i = threadIdx.x; i < LV; i += blockDim.x) vlut[i] = (_Float16)a.tv.cent[i];
    if constexpr (Gm::VPAIR && !KV)
        for (int i = threadIdx.x; i < 256 * VR; i += blockDim.x) {
            const int e = i / VR;
            const half2v hv = {(_Float16)a.tv.cent[e & 15], (_Float16)a.tv.cent[e >> 4]};
            vlut2[i] = __builtin_bit_cast(uint32_t, hv);
        }
    // the sketch operand: entry e holds +2^12 (fp16 0x6c00) for each set bit i of e and -2^12 for
    // each clear one, in bit order; 4 copies (lane l reads copy l % 4) spread the random lookups of
    // a wave over the banks
    if constexpr (QJL)
        for (int i = threadIdx.x; i < 256 * 4; i += blockDim.x) {
            const uint32_t e = (uint32_t)i >> 2;
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = (((e >> (2 * j)) & 1u) ? 0x6c00u : 0xec00u) | ((((e >> (2 * j + 1)) & 1u) ? 0x6c00u : 0xec00u) << 16);
            sgn8[i] = w;
        }
    __syncthreads();
    if constexpr (FQP) {
        if (a.fused_q) {
            constexpr int PL = D / 64;
            const int G = a.group, m = QJL ? a.tk.m : 0;
            if constexpr (QJL) {
                // p_i = sum_j S_ij q_rot_j in index order, for each row of the group
                if ((int)threadIdx.x < m)
                    for (int r = 0; r < G; ++r) {
                        float acc = 0.0f;
#pragma unroll
                        for (int k = 0; k < D / 8; ++k) {
                            const half8 hs = __builtin_bit_cast(half8, srow[k]);
#pragma unroll
                            for (int u = 0; u < 8; ++u) acc = fmaf((float)hs[u], fq_rot[r * D + 8 * k + u], acc);
                        }
                        fq_p[r * 128 + threadIdx.x] = acc * a.p_scale;
                    }
                __syncthreads();
            }
            const int wv = wave_id(), lane = threadIdx.x & 63;
            if (wv < G) {
                // 2^e with the row's largest entry in [2^13, 2^14) (an all-zero or non-finite row keeps
                // e = 0); hi the nearest fp16, lo the nearest fp16 of the remainder
                float qv[PL], pv[2];
                float mx = 0.0f;
#pragma unroll
                for (int c = 0; c < PL; ++c) {
                    qv[c] = fq_rot[wv * D + PL * lane + c] * a.q_scale;
                    mx = fmaxf(mx, fabsf(qv[c]));
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int i = lane + 64 * c;
                    pv[c] = (QJL && i < m) ? fq_p[wv * 128 + i] : 0.0f;
                    mx = fmaxf(mx, fabsf(pv[c]));
                }
                for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
                const int ex = (int)((f2u(mx) >> 23) & 0xffu);
                const int e = (mx > 0.0f && ex < 255) ? 13 - (ex == 0 ? -126 : ex - 127) : 0;
                _Float16* hrow = fq_h + wv * FQS;
#pragma unroll
                for (int c = 0; c < PL; ++c) {
                    const float sv = __builtin_amdgcn_ldexpf(qv[c], e);
                    const _Float16 h = (_Float16)sv;
                    hrow[PL * lane + c] = h;
                    hrow[D + PL * lane + c] = (_Float16)(sv - (float)h);
                }
                if constexpr (QJL)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int i = lane + 64 * c;
                        const float sv = __builtin_amdgcn_ldexpf(pv[c], e);
                        const _Float16 h = (_Float16)sv;
                        if (i < m) {
                            fq_ph[wv * (2 * FQM) + i] = h;
                            fq_ph[wv * (2 * FQM) + FQM + i] = (_Float16)(sv - (float)h);
                        }
                    }
                if (lane == 0) fq_rf[wv] = __builtin_amdgcn_ldexpf(1.0f, -e);
            }
            __syncthreads();
        }
    }

    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const uint8_t* kl = reinterpret_cast<const uint8_t*>(klut) + (lane % KR) * KE;      // the lane's copies
    const uint8_t* vl2 = reinterpret_cast<const uint8_t*>(vlut2) + (lane % VR) * 4;
    const uint8_t* kvl = reinterpret_cast<const uint8_t*>(kvlut);
    const uint8_t* sg8 = reinterpret_cast<const uint8_t*>(sgn8) + (lane & 3) * 16;   // the lane's copies
    const uint32_t koff = 128u + (uint32_t)(lane & 31) * 4u, voff = (uint32_t)(lane & 31) * 4u;
    const uint32_t ksh = (uint32_t)((g * (a.tk.m >> 5)) & 3) * 8u;   // bit offset of the lane's sketch bytes
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_id();
    const int64_t n_streams = (int64_t)a.batch * a.n_kv_heads;
    if (item >= n_streams * a.n_split) return;
    const int64_t st = item / a.n_split;
    const int split = (int)(item - st * a.n_split);
    const int bidx = (int)(st / a.n_kv_heads), kvh = (int)(st - (int64_t)bidx * a.n_kv_heads);
    // this batch element's cache holds `len` valid tokens, shared out over the stream's splits in
    // runs of a multiple of 32 (a split past them stays empty: partials max -inf, sum 0, zero sums,
    // which the combine weighs 0)
    int64_t len = a.n_tokens, tps = a.tokens_per_split;
    if (a.lens) {
        const int64_t l = a.lens[bidx];
        len = l < 0 ? 0 : (l < a.n_tokens ? l : a.n_tokens);
        tps = ((len + a.n_split - 1) / a.n_split + 31) / 32 * 32;
    }
    const int64_t t_begin = (int64_t)split * tps;
    const int64_t t_end = t_begin + tps < len ? t_begin + tps : len;
    const int m = a.tk.m;
    const int mks = m >> 5;

    // query operands (B of the score products): lane column q = l16, k-block g (with PQ, column
    // q + 8 carries query q's lo parts in qb, and qbl is not used)
    const bool qvalid = l16 < a.group;
    const int qcol = PQ ? (l16 & 7) : l16;
    const bool qload = qcol < a.group;
    const int64_t qrow = (int64_t)bidx * a.n_q_heads + (int64_t)kvh * a.group + (qload ? qcol : 0);
    half8 qb[KS], qbl[KS], pb[QJL ? (PQ ? KS : 2 * KS) : 1];   // without PQ, pb[KS + k] the lo parts
    const bool fq = FQP && a.fused_q;
    const int qloc = qload ? qcol : 0;                 // the row within the group
    const float rowf = (fq ? fq_rf[qloc] : a.o.rowf[qrow]) * (1.0f / 4096.0f);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const half8 qh = fq ? *reinterpret_cast<const half8*>(fq_h + qloc * FQS + g * C + 8 * k)
                            : *reinterpret_cast<const half8*>(a.o.qh + qrow * D + g * C + 8 * k);
        const half8 ql = fq ? *reinterpret_cast<const half8*>(fq_h + qloc * FQS + D + g * C + 8 * k)
                            : *reinterpret_cast<const half8*>(a.o.ql + qrow * D + g * C + 8 * k);
        if constexpr (PQ) {
            qb[k] = !qload ? half8{} : (l16 < 8 ? qh : ql);
        } else {
            qb[k] = qvalid ? qh : half8{};
            qbl[k] = qvalid ? ql : half8{};
        }
        if constexpr (QJL) {
            // PQ: columns 8-15 carry the lo parts of the sketch projection, so the sketch term is
            // fp32-accurate like the scores (a sharp softmax amplifies an fp16 rounding of it)
            const bool plo = PQ && l16 >= 8;
            if (k < mks) {
                const int o = g * (m / 4) + 8 * k;
                pb[k] = fq ? *reinterpret_cast<const half8*>(fq_ph + qloc * (2 * FQM) + (plo ? FQM : 0) + o)
                           : *reinterpret_cast<const half8*>((plo ? a.o.pl : a.o.ph) + qrow * m + o);
                if constexpr (!PQ) pb[KS + k] = *reinterpret_cast<const half8*>(a.o.pl + qrow * m + o);
            } else {
                pb[k] = half8{};
                if constexpr (!PQ) pb[KS + k] = half8{};
            }
            if (!qload) pb[k] = half8{};
            if constexpr (!PQ) if (!qload) pb[KS + k] = half8{};
        }
    }

    AttnState<NT> S;
#pragma unroll
    for (int n = 0; n < NT; ++n) S.oacc[n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    S.m_run = -INFINITY;
    S.l_run = 0.0f;

    AttnPtrs P;
    P.kidx = a.pk + a.k_off_idx + st * a.n_tokens * (int64_t)Gm::KROW;
    P.ksk = a.pk + a.k_off_sketch + st * a.n_tokens * (int64_t)(m / 8);
    P.kn = a.pk + a.k_off_norm + st * a.n_tokens * 2;
    P.kr = a.pk + a.k_off_rnorm + st * a.n_tokens * 2;
    P.vidx = a.pv + a.v_off_idx + st * a.n_tokens * (int64_t)Gm::VROW;
    P.vn = a.pv + a.v_off_norm + st * a.n_tokens * 2;
    AttnRes R;
    R.kidx = buffer_rsrc(P.kidx);
    R.ksk = buffer_rsrc(P.ksk);
    R.kn = buffer_rsrc(P.kn);
    R.kr = buffer_rsrc(P.kr);
    R.vidx = buffer_rsrc(P.vidx);
    R.vn = buffer_rsrc(P.vn);
    R.o_kw = (uint32_t)l16 * Gm::KROW + (uint32_t)g * Gm::CBK;
    R.o_ks = (uint32_t)l16 * (uint32_t)(m / 8) + (uint32_t)((g * (m / 32)) & ~3);
    R.o_n = 8u * (uint32_t)g;
    R.o_vw = (uint32_t)(4 * g) * Gm::VROW + (uint32_t)l16 * Gm::VB;

    // full 32-token chunks through two ping-pong buffers (next chunk's loads overlap this one's
    // math), then at most one guarded partial chunk.  Every load in the loop is unconditional (the
    // last refill re-reads the final chunk) so the load counters stay static and a wait covers only
    // the buffer about to be used.
    AttnChunk<Gm::NWK, Gm::NWV, Gm::NKS> A, B;
    const int64_t n_full = t_end > t_begin ? (t_end - t_begin) >> 5 : 0;
    int64_t c = 0;
    if (n_full > 0) {
        attn_load_full<D, BK, BV, QJL>(A, R, t_begin, m);
#pragma unroll 1
        for (; c + 2 <= n_full; c += 2) {
            // (scheduling barriers keep each buffer's loads together, ahead of the other buffer's
            // math, so the wait before a chunk leaves the other buffer's loads in flight)
            attn_load_full<D, BK, BV, QJL>(B, R, t_begin + (c + 1) * 32, m);
            __builtin_amdgcn_sched_barrier(0);
            attn_chunk<D, BK, BV, QJL, true, PQ>(A, S, t_begin + c * 32, t_end, g, mks, qb, qbl, pb, rowf, kl,
                                             vlut, vl2, sg8, kvl, koff, voff, ksh);
            __builtin_amdgcn_sched_barrier(0);
            const int64_t cn = c + 2 < n_full ? c + 2 : n_full - 1;
            attn_load_full<D, BK, BV, QJL>(A, R, t_begin + cn * 32, m);
            __builtin_amdgcn_sched_barrier(0);
            attn_chunk<D, BK, BV, QJL, true, PQ>(B, S, t_begin + (c + 1) * 32, t_end, g, mks, qb, qbl, pb, rowf, kl,
                                             vlut, vl2, sg8, kvl, koff, voff, ksh);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c < n_full) {          // odd count: A holds chunk c
            attn_chunk<D, BK, BV, QJL, true, PQ>(A, S, t_begin + c * 32, t_end, g, mks, qb, qbl, pb, rowf, kl,
                                             vlut, vl2, sg8, kvl, koff, voff, ksh);
            ++c;
        }
    }
    if (t_begin + c * 32 < t_end) {
        attn_load<D, BK, BV, QJL, false>(A, P, t_begin + c * 32, t_end, l16, g, m);
        attn_chunk<D, BK, BV, QJL, false, PQ>(A, S, t_begin + c * 32, t_end, g, mks, qb, qbl, pb, rowf, kl,
                                          vlut, vl2, sg8, kvl, koff, voff, ksh);
    }
    // ---- partial results: lane (q = l16, g) holds O[coord NT*(4g+i) + n][q] --------------------
    const float l_tot = sum4(S.l_run);
    if (qvalid) {
        float* dst = a.part + ((st * a.n_split + split) * 16 + l16) * (int64_t)D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[NT * (4 * g + i) + n] = S.oacc[n][i];
        if (g == 0) {
            float* ml = a.part_ml + ((st * a.n_split + split) * 16 + l16) * 2;
            ml[0] = S.m_run;
            ml[1] = l_tot;
        }
    }
}

// merge the splits of one (batch, q head), rotate back, store.  Latency-bound, so every load is
// issued up front: thread t sums coordinate t % D over the splits s = t / D (mod 256 / D), whose
// partials it fetches before the max is known (16 splits a round); the split maxima and sums go
// through LDS; the first wave applies the inverse rotation s_V ⊙ H(·)/sqrt(d) in registers (lane l
// holds coordinates (D/64) l + c, the low index bits in the lane, the rest as lane-xor butterflies).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    constexpr int NPJ = 256 / D, CH = 16, PL = D / 64;
    const int64_t row = blockIdx.x;                      // batch * n_q_heads + h
    const int bidx = (int)(row / a.n_q_heads), h = (int)(row - (int64_t)bidx * a.n_q_heads);
    const int kvh = h / a.group, r = h - kvh * a.group;
    const int64_t st = (int64_t)bidx * a.n_kv_heads + kvh;
    const int ns = a.n_split, tid = threadIdx.x, lane = tid & 63;
    const int j = tid % D, pj = tid / D;
    __shared__ float buf[D], sums[256], wsp[1024], red[8];   // n_split <= 1024
    const float* ml = a.part_ml + (st * ns * 16 + r) * 2;     // split s at ml[s * 32]
    const float* part = a.part + (st * ns * 16 + r) * (int64_t)D + j;   // split s at part[s * 16 D]
    float pv[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int sp = pj + NPJ * k;
        pv[k] = sp < ns ? part[(int64_t)sp * 16 * D] : 0.0f;
    }
    float mx = -INFINITY;
    for (int sp = tid; sp < ns; sp += 256) mx = fmaxf(mx, ml[sp * 32]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[tid >> 6] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (M == -INFINITY) {                                // an empty cache (length 0): output zeros
        if (tid < D) {
            if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[row * D + tid] = (__bf16)0.0f;
            else reinterpret_cast<float*>(a.out)[row * D + tid] = 0.0f;
        }
        return;
    }
    float ls = 0.0f;
    for (int sp = tid; sp < ns; sp += 256) {
        const float w = exp2f(ml[sp * 32] - M);
        wsp[sp] = w;
        ls += w * ml[sp * 32 + 1];
    }
    for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
    if (lane == 0) red[4 + (tid >> 6)] = ls;
    __syncthreads();
    const float Linv = 1.0f / (red[4] + red[5] + red[6] + red[7]);
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int sp = pj + NPJ * k;
        if (sp < ns) acc = fmaf(wsp[sp], pv[k], acc);
    }
    for (int s0 = NPJ * CH; s0 < ns; s0 += NPJ * CH) {   // more than 16 splits a thread
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int sp = s0 + pj + NPJ * k;
            pv[k] = sp < ns ? part[(int64_t)sp * 16 * D] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int sp = s0 + pj + NPJ * k;
            if (sp < ns) acc = fmaf(wsp[sp], pv[k], acc);
        }
    }
    sums[tid] = acc;
    __syncthreads();
    if (tid < 64) {
        const bool rot = a.tv.rotation != 1;           // Plain-KV values: no inverse rotation
        float v[PL];
#pragma unroll
        for (int c = 0; c < PL; ++c) {
            float t = 0.0f;
#pragma unroll
            for (int q = 0; q < NPJ; ++q) t += sums[q * D + PL * lane + c];
            v[c] = t * Linv;
        }
        if (rot) {
#pragma unroll
            for (int hh = 1; hh < PL; hh <<= 1)
#pragma unroll
                for (int c = 0; c < PL; ++c)
                    if (!(c & hh)) {
                        const float x0 = v[c], x1 = v[c + hh];
                        v[c] = x0 + x1;
                        v[c + hh] = x0 - x1;
                    }
#pragma unroll
            for (int hl = 1; hl < 64; hl <<= 1) {
                const bool hi = (lane & hl) != 0;
#pragma unroll
                for (int c = 0; c < PL; ++c) {
                    const float o = __shfl_xor(v[c], hl);
                    v[c] = hi ? o - v[c] : v[c] + o;
                }
            }
            const float inv = 1.0f / sqrtf((float)D);
            const float* sg = a.tv.signs + (int64_t)kvh * D + PL * lane;
#pragma unroll
            for (int c = 0; c < PL; ++c) v[c] = v[c] * inv * sg[c];
        }
#pragma unroll
        for (int c = 0; c < PL; ++c) {
            const int64_t k = row * D + PL * lane + c;
            if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[k] = (__bf16)v[c];
            else reinterpret_cast<float*>(a.out)[k] = v[c];
        }
    }
}

template <int D, int BK, int BV, bool QJL>
static hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
    const int64_t items = (int64_t)a.batch * a.n_kv_heads * a.n_split;
    if (a.group <= 8) {
        constexpr int threads = attn_threads<D, BK, BV, true>(), waves = threads / 64;
        const int64_t blocks = (items + waves - 1) / waves;
        hipLaunchKernelGGL((attn_kernel<D, BK, BV, QJL, true>), dim3((unsigned)blocks), dim3(threads), 0, s, a);
    } else {
        constexpr int threads = attn_threads<D, BK, BV, false>(), waves = threads / 64;
        const int64_t blocks = (items + waves - 1) / waves;
        hipLaunchKernelGGL((attn_kernel<D, BK, BV, QJL, false>), dim3((unsigned)blocks), dim3(threads), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((int64_t)a.batch * a.n_q_heads)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t launch_db(const AttnArgs& a, hipStream_t s) {
    return a.tk.m > 0 ? launch_one<D, B, B, true>(a, s) : launch_one<D, B, B, false>(a, s);
}

bool attention_fuses_qprep(const AttnArgs& a) {
    // the 768-thread geometry (4-bit keys and values, d <= 128, at most 8 query heads per kv head)
    // with every block's 12 waves on one stream; S rows fit the prep's LDS (m <= 128)
    const int d = a.tk.d;
    if (!(a.tk.b == 4 && a.tv.b == 4 && d <= 128 && a.group <= 8 && a.tk.m <= 128)) return false;
    constexpr int waves = attn_threads<128, 4, 4, true>() / 64;
    static_assert(attn_threads<64, 4, 4, true>() == attn_threads<128, 4, 4, true>(), "one geometry at d <= 128");
    return a.n_split % waves == 0;
}

bool attention_supported(int d, int bk, int bv) {
    // instantiated for b_K == b_V in 2..6; value chunks must be byte aligned per lane: (d/16)·b_V % 8 == 0
    return bk == bv && bk >= 2 && bk <= 6 && ((d / 16) * bv) % 8 == 0;
}

hipError_t launch_attention(const AttnArgs& a, int num_cus, hipStream_t s, bool* supported) {
    (void)num_cus;
    *supported = true;
    const int d = a.tk.d, bk = a.tk.b, bv = a.tv.b;
    if (!attention_supported(d, bk, bv)) {
        *supported = false;
        return hipSuccess;
    }
#define TQ_AT_CASE(DD, BB) \
    if (d == DD && bk == BB) return launch_db<DD, BB>(a, s);
    TQ_AT_CASE(64, 2) TQ_AT_CASE(64, 4) TQ_AT_CASE(64, 6)
    TQ_AT_CASE(128, 2) TQ_AT_CASE(128, 3) TQ_AT_CASE(128, 4) TQ_AT_CASE(128, 5) TQ_AT_CASE(128, 6)
    TQ_AT_CASE(256, 2) TQ_AT_CASE(256, 3) TQ_AT_CASE(256, 4) TQ_AT_CASE(256, 5) TQ_AT_CASE(256, 6)
#undef TQ_AT_CASE
    *supported = false;
    return hipSuccess;
}

}  // namespace tq
