// Fused GQA decode attention over the packed cache ("Ablation, Statistical Inference, and
// Validation for KV-Cache Compression", eq. (1) T = softmax(QK^T/sqrt(d))V, with the scores
// estimated on compressed keys as in §2 TurboQuant / SpectralQuant paragraphs).
//
// Split-K (flash-decoding): one wave per (stream = batch·n_kv + kv head, token split).  Per chunk
// of 32 tokens:
//   scores  D[token][q] = K̂ Q^T on v_mfma_f32_16x16x32_f16 (A = dequantised keys, lane = token
//           l%16 with its packed k-block l/16; B = fp16 rotated queries), plus the QJL term
//           <p, 2σ-1> with A = ±1 sketch bits and B = fp16 S·q_rot;
//   softmax online in base 2; the score accumulator of lane (q = l%16, g = l/16) holds tokens
//           {4g+i, 16+4g+i}, exactly the k-block g of the B operand of the next product;
//   values  O^T[coord][q] += V̂^T W^T (A = dequantised values, lane = coordinate row l%16 over its
//           8 tokens), accumulated in the rotated domain — no per-token inverse transform.
// A combine kernel merges the splits and applies the inverse rotation s_V ⊙ H(·)/sqrt(d) once.
#include "common.hpp"
#include "kernels.hpp"

namespace tq {

__device__ __forceinline__ float max4(float t) {
    float a = t, b = t;
    xswap16(a, b);
    t = fmaxf(a, b);
    a = t;
    b = t;
    xswap32(a, b);
    return fmaxf(a, b);
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
    static constexpr int KE = 2 * PK;                // bytes per K LUT entry
    static constexpr int KR = (NEK * KE * (128 / KE) <= 32768) ? 128 / KE : 1;
    static constexpr int VR = VPAIR ? 32 : 1;        // copies of the 1 KiB value pair LUT
    // 4-bit keys and values: both LUTs have 256 entries of 4 bytes, so one table of 256-byte rows
    // holds entry e of both (32 K copies, then 32 V copies), and a lane's address is the byte
    // index shifted by 8 or-ed with its copy offset: one v_perm_b32 per lookup.
    static constexpr bool KV256 = VPAIR && PK == 2 && NEK == 256;
};

// byte offset (idx << 8) | off, idx = byte `which` of w, off < 256: D = {0, 0, w.byte[which], off.byte0}
__device__ __forceinline__ uint32_t row256(uint32_t w, uint32_t off, int which) {
    return __builtin_amdgcn_perm(w, off, 0x0c0c0000u | ((uint32_t)(4 + which) << 8));
}

// Per-wave base pointers of one stream (chunk offsets are added as wave-uniform values).
struct AttnPtrs {
    const uint8_t* kidx;
    const uint8_t* ksk;
    const uint8_t* kn;
    const uint8_t* kr;
    const uint8_t* vidx;
    const uint8_t* vn;
};

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

template <int D, int BK, int BV, bool QJL, bool FULL>
__device__ __forceinline__ void attn_chunk(const AttnChunk<AttnGeom<D, BK, BV>::NWK, AttnGeom<D, BK, BV>::NWV, AttnGeom<D, BK, BV>::NKS>& cur,
                                           AttnState<AttnGeom<D, BK, BV>::NT>& S, int64_t t0, int64_t t_end,
                                           int g, int mks,
                                           const half8 (&qb)[AttnGeom<D, BK, BV>::KS], const half8* pb,
                                           const uint8_t* kl, const _Float16* vlut, const uint8_t* vl2,
                                           const u32x2* sgn4, const uint8_t* kvl, uint32_t koff, uint32_t voff,
                                           uint32_t ksh) {
    using Gm = AttnGeom<D, BK, BV>;
    constexpr int KS = Gm::KS, PK = Gm::PK, NT = Gm::NT;
    // ---- scores for the two 16-token tiles ----------------------------------------------------
    float lg[8];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        half8 ka[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            constexpr int KST = Gm::KR * Gm::KE;      // bytes between entries of one copy
            if constexpr (PK == 8) {
                const uint32_t f = get_bits<8 * BK>(cur.kw[T], (8 * k) * BK);
                ka[k] = *reinterpret_cast<const half8*>(kl + f * KST);
            } else if constexpr (PK == 4) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t f = get_bits<4 * BK>(cur.kw[T], (8 * k + 4 * h) * BK);
                    const half4 e = *reinterpret_cast<const half4*>(kl + f * KST);
                    ka[k][4 * h + 0] = e[0]; ka[k][4 * h + 1] = e[1];
                    ka[k][4 * h + 2] = e[2]; ka[k][4 * h + 3] = e[3];
                }
            } else if constexpr (Gm::KV256) {
                // coordinates (8k + 2h, +1) are byte h of packed word k
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const half2v e = *reinterpret_cast<const half2v*>(kvl + row256(cur.kw[T][k], koff, h));
                    ka[k][2 * h] = e[0];
                    ka[k][2 * h + 1] = e[1];
                }
            } else if constexpr (PK == 2) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t f = get_bits<2 * BK>(cur.kw[T], (8 * k + 2 * h) * BK);
                    const half2v e = *reinterpret_cast<const half2v*>(kl + f * KST);
                    ka[k][2 * h] = e[0];
                    ka[k][2 * h + 1] = e[1];
                }
            } else {
#pragma unroll
                for (int h = 0; h < 8; ++h)
                    ka[k][h] = *reinterpret_cast<const _Float16*>(kl + get_bits<BK>(cur.kw[T], (8 * k + h) * BK) * KST);
            }
        }
        floatx4 s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KS; ++k) s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[k], qb[k], s1, 0, 0, 0);
        floatx4 s2 = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (QJL) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if (k < mks) {
                    const uint32_t wsk = __builtin_amdgcn_alignbit(cur.ks[T][(k >> 2) + 1], cur.ks[T][k >> 2], ksh);
                    const u32x2 lo = sgn4[(wsk >> (8 * (k & 3))) & 0xfu];
                    const u32x2 hi = sgn4[(wsk >> (8 * (k & 3) + 4)) & 0xfu];
                    const half8 sa = __builtin_bit_cast(half8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    s2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, pb[k], s2, 0, 0, 0);
                }
            }
        }
        // output lane (q = l16, g) holds tokens t0 + 16T + 4g + i; the queries (and their sketch
        // projections) already carry the softmax scale in log2 units (and sqrt(pi/2)/m), so the
        // base-2 logit is n16 (s1 + r16 s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sc = s1[i];
            if constexpr (QJL) sc = fmaf(half_of(cur.kr[T], i), s2[i], sc);
            float v = half_of(cur.kn[T], i) * sc;
            if (!FULL && t0 + 16 * T + 4 * g + i >= t_end) v = -INFINITY;
            lg[4 * T + i] = v;
        }
    }
    // ---- online softmax (base 2) per query column; rescale only when a running max moved ---------
    float cmax = lg[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, lg[r]);
    cmax = max4(cmax);
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
    for (int r = 0; r < 8; ++r) {
        const _Float16 wh = (_Float16)__builtin_amdgcn_exp2f(lg[r] - m_new);
        wsum += (float)wh;
        wb[r] = wh * (_Float16)half_of(cur.vn[r >> 2], r & 3);
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
                ze[p] = (w0 & 0x0f0f0f0fu) | ((w1 << 4) & 0xf0f0f0f0u);
                zo[p] = ((w0 >> 4) & 0x0f0f0f0fu) | (w1 & 0xf0f0f0f0u);
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

template <int D, int BK, int BV, bool QJL>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void attn_kernel(AttnArgs a) {
    using Gm = AttnGeom<D, BK, BV>;
    constexpr int C = Gm::C, KS = Gm::KS, PK = Gm::PK, NEK = Gm::NEK, NT = Gm::NT;
    constexpr int LV = 1 << BV;

    constexpr int KR = Gm::KR, KE = Gm::KE, VR = Gm::VR;
    constexpr bool KV = Gm::KV256;
    __shared__ uint32_t klut[KV ? 1 : NEK * KE / 4 * KR];          // copy c of entry e at (e KR + c) KE bytes
    __shared__ _Float16 vlut[LV];
    __shared__ uint32_t vlut2[Gm::VPAIR && !KV ? 256 * VR : 1];  // copy c of entry e at word e VR + c
    __shared__ uint32_t kvlut[KV ? 256 * 64 : 1];                 // row e: 32 K copies, 32 V copies
    __shared__ u32x2 sgn4[16];                                     // ±1 halves of the 4 bits of a nibble
    if constexpr (KV) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.tk.lut_f16);
        for (int i = threadIdx.x; i < 256 * 64; i += blockDim.x) {
            const int e = i >> 6, c = i & 63;
            if (c < 32) {
                kvlut[i] = src[e];
            } else {
                const half2v hv = {(_Float16)a.tv.cent[e & 15], (_Float16)a.tv.cent[e >> 4]};
                kvlut[i] = __builtin_bit_cast(uint32_t, hv);
            }
        }
    } else {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(a.tk.lut_f16);
        uint16_t* dst = reinterpret_cast<uint16_t*>(klut);
        for (int i = threadIdx.x; i < NEK * KR; i += blockDim.x) {
            const int e = i / KR, c = i - e * KR;
#pragma unroll
            for (int h = 0; h < PK; ++h) dst[(e * KR + c) * PK + h] = src[e * PK + h];
        }
    }
    for (int i = threadIdx.x; i < LV; i += blockDim.x) vlut[i] = (_Float16)a.tv.cent[i];
    if constexpr (Gm::VPAIR && !KV)
        for (int i = threadIdx.x; i < 256 * VR; i += blockDim.x) {
            const int e = i / VR;
            const half2v hv = {(_Float16)a.tv.cent[e & 15], (_Float16)a.tv.cent[e >> 4]};
            vlut2[i] = __builtin_bit_cast(uint32_t, hv);
        }
    if (threadIdx.x < 16) {
        uint32_t w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            w[j] = (((threadIdx.x >> (2 * j)) & 1) ? 0x3c00u : 0xbc00u) |
                   ((((threadIdx.x >> (2 * j + 1)) & 1) ? 0x3c00u : 0xbc00u) << 16);
        sgn4[threadIdx.x] = u32x2{w[0], w[1]};
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const uint8_t* kl = reinterpret_cast<const uint8_t*>(klut) + (lane % KR) * KE;      // the lane's copies
    const uint8_t* vl2 = reinterpret_cast<const uint8_t*>(vlut2) + (lane % VR) * 4;
    const uint8_t* kvl = reinterpret_cast<const uint8_t*>(kvlut);
    const uint32_t koff = (uint32_t)(lane & 31) * 4u, voff = 128u + (uint32_t)(lane & 31) * 4u;
    const uint32_t ksh = (uint32_t)((g * (a.tk.m >> 5)) & 3) * 8u;   // bit offset of the lane's sketch bytes
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
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

    // query operands (B of the score products): lane column q = l16, k-block g
    const bool qvalid = l16 < a.group;
    const int64_t qrow = (int64_t)bidx * a.n_q_heads + (int64_t)kvh * a.group + (qvalid ? l16 : 0);
    half8 qb[KS], pb[QJL ? KS : 1];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        qb[k] = *reinterpret_cast<const half8*>(a.q_rot + qrow * D + g * C + 8 * k);
        if (!qvalid) qb[k] = half8{};
        if constexpr (QJL) {
            if (k < mks) pb[k] = *reinterpret_cast<const half8*>(a.p + qrow * m + g * (m / 4) + 8 * k);
            else pb[k] = half8{};
            if (!qvalid) pb[k] = half8{};
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

    // full 32-token chunks through two ping-pong buffers (next chunk's loads overlap this one's
    // math), then at most one guarded partial chunk.  Every load in the loop is unconditional (the
    // last refill re-reads the final chunk) so the load counters stay static and a wait covers only
    // the buffer about to be used.
    AttnChunk<Gm::NWK, Gm::NWV, Gm::NKS> A, B;
    const int64_t n_full = t_end > t_begin ? (t_end - t_begin) >> 5 : 0;
    int64_t c = 0;
    if (n_full > 0) {
        attn_load<D, BK, BV, QJL, true>(A, P, t_begin, t_end, l16, g, m);
#pragma unroll 1
        for (; c + 2 <= n_full; c += 2) {
            // (scheduling barriers keep each buffer's loads together, ahead of the other buffer's
            // math, so the wait before a chunk leaves the other buffer's loads in flight)
            attn_load<D, BK, BV, QJL, true>(B, P, t_begin + (c + 1) * 32, t_end, l16, g, m);
            __builtin_amdgcn_sched_barrier(0);
            attn_chunk<D, BK, BV, QJL, true>(A, S, t_begin + c * 32, t_end, g, mks, qb, pb, kl,
                                             vlut, vl2, sgn4, kvl, koff, voff, ksh);
            __builtin_amdgcn_sched_barrier(0);
            const int64_t cn = c + 2 < n_full ? c + 2 : n_full - 1;
            attn_load<D, BK, BV, QJL, true>(A, P, t_begin + cn * 32, t_end, l16, g, m);
            __builtin_amdgcn_sched_barrier(0);
            attn_chunk<D, BK, BV, QJL, true>(B, S, t_begin + (c + 1) * 32, t_end, g, mks, qb, pb, kl,
                                             vlut, vl2, sgn4, kvl, koff, voff, ksh);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c < n_full) {          // odd count: A holds chunk c
            attn_chunk<D, BK, BV, QJL, true>(A, S, t_begin + c * 32, t_end, g, mks, qb, pb, kl,
                                             vlut, vl2, sgn4, kvl, koff, voff, ksh);
            ++c;
        }
    }
    if (t_begin + c * 32 < t_end) {
        attn_load<D, BK, BV, QJL, false>(A, P, t_begin + c * 32, t_end, l16, g, m);
        attn_chunk<D, BK, BV, QJL, false>(A, S, t_begin + c * 32, t_end, g, mks, qb, pb, kl,
                                          vlut, vl2, sgn4, kvl, koff, voff, ksh);
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

// merge the splits of one (batch, q head), rotate back, store
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int64_t row = blockIdx.x;                      // batch * n_q_heads + h
    const int bidx = (int)(row / a.n_q_heads), h = (int)(row - (int64_t)bidx * a.n_q_heads);
    const int kvh = h / a.group, r = h - kvh * a.group;
    const int64_t st = (int64_t)bidx * a.n_kv_heads + kvh;
    const int d = a.tv.d, ns = a.n_split;
    __shared__ float buf[256];
    __shared__ float wsp[1024];                          // per-split weights (n_split <= 1024)
    __shared__ float red[8];
    const float* ml = a.part_ml + (st * ns * 16 + r) * 2;   // split s at ml[s * 32]
    // max over splits
    float mx = -INFINITY;
    for (int s = threadIdx.x; s < ns; s += blockDim.x) mx = fmaxf(mx, ml[s * 32]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (M == -INFINITY) {                                // an empty cache (length 0): output zeros
        for (int j = threadIdx.x; j < d; j += blockDim.x) {
            if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[row * d + j] = (__bf16)0.0f;
            else reinterpret_cast<float*>(a.out)[row * d + j] = 0.0f;
        }
        return;
    }
    float ls = 0.0f;
    for (int s = threadIdx.x; s < ns; s += blockDim.x) {
        const float w = exp2f(ml[s * 32] - M);
        wsp[s] = w;
        ls += w * ml[s * 32 + 1];
    }
    for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[4 + (threadIdx.x >> 6)] = ls;
    __syncthreads();
    const float Linv = 1.0f / (red[4] + red[5] + red[6] + red[7]);
    const float* part = a.part + (st * ns * 16 + r) * (int64_t)d;  // split s at part[s * 16 d]
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        float acc0 = 0.0f, acc1 = 0.0f, acc2 = 0.0f, acc3 = 0.0f;
        int s = 0;
        for (; s + 4 <= ns; s += 4) {
            acc0 = fmaf(wsp[s], part[(int64_t)s * 16 * d + j], acc0);
            acc1 = fmaf(wsp[s + 1], part[(int64_t)(s + 1) * 16 * d + j], acc1);
            acc2 = fmaf(wsp[s + 2], part[(int64_t)(s + 2) * 16 * d + j], acc2);
            acc3 = fmaf(wsp[s + 3], part[(int64_t)(s + 3) * 16 * d + j], acc3);
        }
        for (; s < ns; ++s) acc0 = fmaf(wsp[s], part[(int64_t)s * 16 * d + j], acc0);
        buf[j] = ((acc0 + acc1) + (acc2 + acc3)) * Linv;
    }
    __syncthreads();
    const bool rot = a.tv.rotation != 1;               // Plain-KV values: no inverse rotation
    for (int hh = 1; hh < (rot ? d : 1); hh <<= 1) {
        for (int i = threadIdx.x; i < d / 2; i += blockDim.x) {
            const int lo = (i / hh) * 2 * hh + (i % hh);
            const float x0 = buf[lo], x1 = buf[lo + hh];
            buf[lo] = x0 + x1;
            buf[lo + hh] = x0 - x1;
        }
        __syncthreads();
    }
    const float inv = rot ? 1.0f / sqrtf((float)d) : 1.0f;
    const float* sg = a.tv.signs + (int64_t)kvh * d;
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        const float o = rot ? buf[j] * inv * sg[j] : buf[j];
        if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[row * d + j] = (__bf16)o;
        else reinterpret_cast<float*>(a.out)[row * d + j] = o;
    }
}

template <int D, int BK, int BV, bool QJL>
static hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
    const int64_t items = (int64_t)a.batch * a.n_kv_heads * a.n_split;
    const int64_t blocks = (items + 3) / 4;
    hipLaunchKernelGGL((attn_kernel<D, BK, BV, QJL>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((int64_t)a.batch * a.n_q_heads)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t launch_db(const AttnArgs& a, hipStream_t s) {
    return a.tk.m > 0 ? launch_one<D, B, B, true>(a, s) : launch_one<D, B, B, false>(a, s);
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
