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
template <int NWK, int NWV>
struct AttnChunk {
    uint32_t kw[2][NWK];
    uint32_t ks[2][2];
    u32x2 kn[2], kr[2], vn[2];
    uint32_t vw[8][NWV];
};

__device__ __forceinline__ int64_t tau_tok(int g, int r) { return r < 4 ? 4 * g + r : 16 + 4 * g + (r - 4); }

template <int D, int BK, int BV, bool QJL, int NWK, int NWV>
__device__ __forceinline__ void attn_load(AttnChunk<NWK, NWV>& c, int64_t t0, int64_t t_end, int l16, int g, int m,
                                          const uint8_t* kidx, const uint8_t* ksk, const _Float16* kn,
                                          const _Float16* kr, const uint8_t* vidx, const _Float16* vn) {
    constexpr int C = D / 4;
    constexpr int CBK = C * BK / 8, CAK = cmin(pow2_align(CBK), 16);
    constexpr int NT = D / 16, VB = NT * BV / 8, VA = cmin(pow2_align(VB), 16);
    const bool full = t0 + 32 <= t_end;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        const int64_t tk = t0 + 16 * T + l16;
        if (full || tk < t_end) {
            load_bytes<CBK, CAK>(kidx + tk * (D * BK / 8) + g * CBK, c.kw[T]);
            if constexpr (QJL) {
                const uint8_t* sp = ksk + tk * (m / 8) + g * (m / 32);
                if ((m & 127) == 0) {
                    c.ks[T][0] = *reinterpret_cast<const uint32_t*>(sp);
                    c.ks[T][1] = m == 256 ? *reinterpret_cast<const uint32_t*>(sp + 4) : 0u;
                } else {
                    uint32_t w0 = 0, w1 = 0;
                    for (int q = 0; q < (m >> 5); ++q) {
                        if (q < 4) w0 |= uint32_t(sp[q]) << (8 * q);
                        else w1 |= uint32_t(sp[q]) << (8 * (q - 4));
                    }
                    c.ks[T][0] = w0;
                    c.ks[T][1] = w1;
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < NWK; ++k) c.kw[T][k] = 0u;
            c.ks[T][0] = c.ks[T][1] = 0u;
        }
        const int64_t tn = t0 + 16 * T + 4 * g;   // 4 consecutive tokens, 8-byte aligned
        if (full || tn + 4 <= t_end) {
            c.kn[T] = *reinterpret_cast<const u32x2*>(kn + tn);
            if constexpr (QJL) c.kr[T] = *reinterpret_cast<const u32x2*>(kr + tn);
            c.vn[T] = *reinterpret_cast<const u32x2*>(vn + tn);
        } else {
            uint32_t a[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0}, e[4] = {0, 0, 0, 0};
            for (int i = 0; i < 4; ++i)
                if (tn + i < t_end) {
                    a[i] = *reinterpret_cast<const uint16_t*>(kn + tn + i);
                    if constexpr (QJL) b[i] = *reinterpret_cast<const uint16_t*>(kr + tn + i);
                    e[i] = *reinterpret_cast<const uint16_t*>(vn + tn + i);
                }
            c.kn[T] = u32x2{a[0] | (a[1] << 16), a[2] | (a[3] << 16)};
            c.kr[T] = u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
            c.vn[T] = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t tt = t0 + tau_tok(g, r);
        if (full || tt < t_end) load_bytes<VB, VA>(vidx + tt * (D * BV / 8) + l16 * VB, c.vw[r]);
        else {
#pragma unroll
            for (int k = 0; k < NWV; ++k) c.vw[r][k] = 0u;
        }
    }
}

__device__ __forceinline__ float half_of(const u32x2& v, int i) {
    const uint32_t w = v[i >> 1];
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
}

template <int D, int BK, int BV, bool QJL>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    constexpr int C = D / 4;
    constexpr int KS = C / 8;                       // k-steps over d
    constexpr int PK = lut_group_c(BK), NEK = 1 << (PK * BK);
    constexpr int NWK = (C * BK + 31) / 32;
    constexpr int NT = D / 16;                      // value tiles (16 coordinates each)
    constexpr int NWV = (NT * BV + 31) / 32;
    constexpr int LV = 1 << BV;

    __shared__ _Float16 klut[NEK * PK];
    __shared__ _Float16 vlut[LV];
    __shared__ _Float16 sgn[QJL ? 256 * 8 : 8];
    for (int i = threadIdx.x; i < NEK * PK; i += blockDim.x) klut[i] = a.tk.lut_f16[i];
    for (int i = threadIdx.x; i < LV; i += blockDim.x) vlut[i] = (_Float16)a.tv.cent[i];
    if constexpr (QJL)
        for (int i = threadIdx.x; i < 256; i += blockDim.x)
#pragma unroll
            for (int k = 0; k < 8; ++k) sgn[i * 8 + k] = ((i >> k) & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t n_streams = (int64_t)a.batch * a.n_kv_heads;
    if (item >= n_streams * a.n_split) return;
    const int64_t st = item / a.n_split;
    const int split = (int)(item - st * a.n_split);
    const int64_t t_begin = (int64_t)split * a.tokens_per_split;
    const int64_t t_end = t_begin + a.tokens_per_split < a.n_tokens ? t_begin + a.tokens_per_split : a.n_tokens;
    const int m = a.tk.m;
    const int mks = m >> 5;
    const float lam = QJL ? 1.2533141373155003f / (float)m : 0.0f;

    // query operands (B of the score products): lane column q = l16, k-block g
    const int bidx = (int)(st / a.n_kv_heads), kvh = (int)(st - (int64_t)bidx * a.n_kv_heads);
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

    floatx4 oacc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    const uint8_t* kidx = a.pk + a.k_off_idx + st * a.n_tokens * (int64_t)(D * BK / 8);
    const uint8_t* ksk = a.pk + a.k_off_sketch + st * a.n_tokens * (int64_t)(m / 8);
    const _Float16* kn = reinterpret_cast<const _Float16*>(a.pk + a.k_off_norm) + st * a.n_tokens;
    const _Float16* kr = reinterpret_cast<const _Float16*>(a.pk + a.k_off_rnorm) + st * a.n_tokens;
    const uint8_t* vidx = a.pv + a.v_off_idx + st * a.n_tokens * (int64_t)(D * BV / 8);
    const _Float16* vn = reinterpret_cast<const _Float16*>(a.pv + a.v_off_norm) + st * a.n_tokens;

    AttnChunk<NWK, NWV> nxt;
    attn_load<D, BK, BV, QJL>(nxt, t_begin, t_end, l16, g, m, kidx, ksk, kn, kr, vidx, vn);
#pragma unroll 1
    for (int64_t t0 = t_begin; t0 < t_end; t0 += 32) {
        const AttnChunk<NWK, NWV> cur = nxt;
        if (t0 + 32 < t_end)   // issue the next chunk's loads before computing this one
            attn_load<D, BK, BV, QJL>(nxt, t0 + 32, t_end, l16, g, m, kidx, ksk, kn, kr, vidx, vn);
        const bool full = t0 + 32 <= t_end;
        // ---- scores for the two 16-token tiles ----------------------------------------------
        float lg[8];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            half8 ka[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if constexpr (PK == 8) {
                    const uint32_t f = get_bits<8 * BK>(cur.kw[T], (8 * k) * BK);
                    ka[k] = *reinterpret_cast<const half8*>(klut + f * 8);
                } else if constexpr (PK == 4) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t f = get_bits<4 * BK>(cur.kw[T], (8 * k + 4 * h) * BK);
                        const half4 e = *reinterpret_cast<const half4*>(klut + f * 4);
                        ka[k][4 * h + 0] = e[0]; ka[k][4 * h + 1] = e[1];
                        ka[k][4 * h + 2] = e[2]; ka[k][4 * h + 3] = e[3];
                    }
                } else if constexpr (PK == 2) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t f = get_bits<2 * BK>(cur.kw[T], (8 * k + 2 * h) * BK);
                        const half2v e = *reinterpret_cast<const half2v*>(klut + f * 2);
                        ka[k][2 * h] = e[0];
                        ka[k][2 * h + 1] = e[1];
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < 8; ++h) ka[k][h] = klut[get_bits<BK>(cur.kw[T], (8 * k + h) * BK)];
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
                        const uint32_t byte = (cur.ks[T][k >> 2] >> (8 * (k & 3))) & 0xffu;
                        const half8 sa = *reinterpret_cast<const half8*>(sgn + byte * 8);
                        s2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, pb[k], s2, 0, 0, 0);
                    }
                }
            }
            // output lane (q = l16, g) holds tokens t0 + 16T + 4g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sc = s1[i];
                if constexpr (QJL) sc = fmaf(lam * half_of(cur.kr[T], i), s2[i], sc);
                float v = half_of(cur.kn[T], i) * sc * a.scale_log2;
                if (!full && t0 + 16 * T + 4 * g + i >= t_end) v = -INFINITY;
                lg[4 * T + i] = v;
            }
        }
        // ---- online softmax (base 2) per query column -----------------------------------------
        float cmax = lg[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, lg[r]);
        cmax = max4(cmax);
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float wsum = 0.0f;
        half8 wb;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float w = exp2f(lg[r] - m_new);
            const _Float16 wh = (_Float16)w;
            wsum += (float)wh;
            wb[r] = (_Float16)((float)wh * half_of(cur.vn[r >> 2], r & 3));
        }
        l_run = l_run * alpha + wsum;
#pragma unroll
        for (int n = 0; n < NT; ++n) oacc[n] *= alpha;
        // ---- values: A = V̂^T tile n (row = coordinate NT*l16 + n), 8 tokens of k-block g ---------
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            half8 va;
#pragma unroll
            for (int r = 0; r < 8; ++r) va[r] = vlut[get_bits<BV>(cur.vw[r], n * BV)];
            oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, wb, oacc[n], 0, 0, 0);
        }
    }
    // ---- partial results: lane (q = l16, g) holds O[coord NT*(4g+i) + n][q] --------------------
    l_run = sum4(l_run);
    if (qvalid) {
        float* dst = a.part + ((st * a.n_split + split) * 16 + l16) * (int64_t)D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[NT * (4 * g + i) + n] = oacc[n][i];
        if (g == 0) {
            float* ml = a.part_ml + ((st * a.n_split + split) * 16 + l16) * 2;
            ml[0] = m_run;
            ml[1] = l_run;
        }
    }
}

// merge the splits of one (batch, q head), rotate back, store
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int64_t row = blockIdx.x;                      // batch * n_q_heads + h
    const int bidx = (int)(row / a.n_q_heads), h = (int)(row - (int64_t)bidx * a.n_q_heads);
    const int kvh = h / a.group, r = h - kvh * a.group;
    const int64_t st = (int64_t)bidx * a.n_kv_heads + kvh;
    const int d = a.tv.d;
    __shared__ float buf[256];
    __shared__ float red[2];
    if (threadIdx.x == 0) {
        float M = -INFINITY;
        for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_ml[((st * a.n_split + s) * 16 + r) * 2]);
        float Lsum = 0.0f;
        for (int s = 0; s < a.n_split; ++s) {
            const float* ml = a.part_ml + ((st * a.n_split + s) * 16 + r) * 2;
            Lsum += ml[1] * exp2f(ml[0] - M);
        }
        red[0] = M;
        red[1] = Lsum;
    }
    __syncthreads();
    const float M = red[0], Linv = 1.0f / red[1];
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        float acc = 0.0f;
        for (int s = 0; s < a.n_split; ++s) {
            const float wgt = exp2f(a.part_ml[((st * a.n_split + s) * 16 + r) * 2] - M);
            acc = fmaf(wgt, a.part[((st * a.n_split + s) * 16 + r) * (int64_t)d + j], acc);
        }
        buf[j] = acc * Linv;
    }
    __syncthreads();
    for (int hh = 1; hh < d; hh <<= 1) {
        for (int i = threadIdx.x; i < d / 2; i += blockDim.x) {
            const int lo = (i / hh) * 2 * hh + (i % hh);
            const float x0 = buf[lo], x1 = buf[lo + hh];
            buf[lo] = x0 + x1;
            buf[lo + hh] = x0 - x1;
        }
        __syncthreads();
    }
    const float inv = 1.0f / sqrtf((float)d);
    const float* sg = a.tv.signs + (int64_t)kvh * d;
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        const float o = buf[j] * inv * sg[j];
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
