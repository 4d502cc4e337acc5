// Query preparation and score estimation on packed keys ("Ablation, Statistical Inference, and
// Validation for KV-Cache Compression", §2: TurboQuant paragraph — QJL on K improves the score
// estimate <q,k>; SpectralQuant paragraph — the asymmetric 1-bit estimator; here in the WHT domain
// with a Gaussian S):
//   q_rot = H (q ⊙ s) / sqrt(d),  p = S q_rot,
//   ŝ(q, k) = n16 · ( <q_rot, c[idx]> + sqrt(pi/2)/m · r16 · <p, 2σ - 1> ).
// The two contractions over d and m are v_mfma_f32_16x16x32_f16 tiles: A = 16 queries (fp16
// q_rot / p), B = 16 keys dequantised straight from the packed bytes.  Lane l holds key l%16 and the
// k-block l/16, which is exactly the contiguous packed chunk g = l/16 the encoder wrote.
#include "common.hpp"
#include "kernels.hpp"

namespace tq {

// ---------------------------------------------------------------------------------------------
// q_rot and p per query row; one block of 256 threads per row (tiny amount of work).
__global__ __launch_bounds__(256) void qprep_kernel(QPrepArgs a) {
    const int64_t row = blockIdx.x;
    const int d = a.t.d, m = a.t.m;
    const int head = (int)((row / a.n_q_per_stream) % a.t.n_heads);
    __shared__ float buf[256];
    const float* sg = a.t.signs + (int64_t)head * d;
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        float x;
        if (a.q_bf16) {
            const uint16_t u = reinterpret_cast<const uint16_t*>(a.q)[row * d + j];
            x = u2f(uint32_t(u) << 16);
        } else {
            x = reinterpret_cast<const float*>(a.q)[row * d + j];
        }
        buf[j] = x * sg[j];
    }
    __syncthreads();
    for (int h = 1; h < d; h <<= 1) {
        for (int i = threadIdx.x; i < d / 2; i += blockDim.x) {
            const int lo = (i / h) * 2 * h + (i % h);
            const float x0 = buf[lo], x1 = buf[lo + h];
            buf[lo] = x0 + x1;
            buf[lo + h] = x0 - x1;
        }
        __syncthreads();
    }
    const float inv = 1.0f / sqrtf((float)d);
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        const float r = buf[j] * inv;
        buf[j] = r;
        a.q_rot[row * d + j] = (_Float16)(r * a.q_scale);
    }
    __syncthreads();
    if (m > 0) {
        const _Float16* S = a.t.S + (int64_t)head * m * d;
        for (int i = threadIdx.x; i < m; i += blockDim.x) {
            float acc = 0.0f;
            for (int j = 0; j < d; ++j) acc = fmaf((float)S[(int64_t)i * d + j], buf[j], acc);
            a.p[row * m + i] = (_Float16)(acc * a.p_scale);
        }
    }
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s) {
    if (a.n_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)a.n_rows), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Dequantise the lane's C packed coordinates into C/8 fp16x8 MFMA operands.
template <int C, int B>
__device__ __forceinline__ void dequant_f16(const uint32_t (&w)[(C * B + 31) / 32], const _Float16* lut,
                                            half8 (&out)[C / 8]) {
    constexpr int P = lut_group_c(B);
#pragma unroll
    for (int k = 0; k < C / 8; ++k) {
        if constexpr (P == 8) {
            const uint32_t f = get_bits<8 * B>(w, (8 * k) * B);
            out[k] = *reinterpret_cast<const half8*>(lut + f * 8);
        } else if constexpr (P == 4) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t f = get_bits<4 * B>(w, (8 * k + 4 * h) * B);
                const half4 e = *reinterpret_cast<const half4*>(lut + f * 4);
                out[k][4 * h + 0] = e[0]; out[k][4 * h + 1] = e[1];
                out[k][4 * h + 2] = e[2]; out[k][4 * h + 3] = e[3];
            }
        } else if constexpr (P == 2) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t f = get_bits<2 * B>(w, (8 * k + 2 * h) * B);
                const half2v e = *reinterpret_cast<const half2v*>(lut + f * 2);
                out[k][2 * h] = e[0];
                out[k][2 * h + 1] = e[1];
            }
        } else {
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const uint32_t f = get_bits<B>(w, (8 * k + h) * B);
                out[k][h] = lut[f];
            }
        }
    }
}

// 256 x 8 fp16 table: byte -> (+1 if bit set else -1) for its 8 bits, LSB first
__device__ __forceinline__ void build_sign_lut(_Float16* t) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x)
#pragma unroll
        for (int k = 0; k < 8; ++k) t[i * 8 + k] = ((i >> k) & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
}

template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) void scores_kernel(ScoresArgs a) {
    constexpr int C = D / 4;
    constexpr int P = lut_group_c(B), NE = 1 << (P * B);
    constexpr int NW = (C * B + 31) / 32;
    constexpr int CB = C * B / 8;
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr int KS = C / 8;                   // k-steps over d (and the maximum over m <= d)

    __shared__ _Float16 lut[NE * P];
    __shared__ _Float16 sgn[QJL ? 256 * 8 : 8];
    for (int i = threadIdx.x; i < NE * P; i += blockDim.x) lut[i] = a.t.lut_f16[i];
    if constexpr (QJL) build_sign_lut(sgn);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int t16 = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const int64_t st = blockIdx.x / a.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int m = a.t.m;
    const int mks = m >> 5;                     // sketch k-steps (m/4 bits per lane, 8 per step)
    const float lam = QJL ? 1.2533141373155003f / (float)m : 0.0f;   // sqrt(pi/2)/m
    const int nqt = (a.n_q + 15) >> 4;

#pragma unroll 1
    for (int64_t tile = tb0 + wave; tile < tb1; tile += 4) {
        const int64_t tok = tile * 16 + t16;
        const bool valid = tok < a.n_tokens;
        const int64_t vec = st * a.n_tokens + (valid ? tok : 0);
        uint32_t w[NW];
        float n16 = 0.0f, r16 = 0.0f;
        if (valid) {
            load_bytes<CB, CA>(a.packed + a.off_idx + vec * (int64_t)(D * B / 8) + g * CB, w);
            n16 = (float)*reinterpret_cast<const _Float16*>(a.packed + a.off_norm + vec * 2);
            if constexpr (QJL) r16 = (float)*reinterpret_cast<const _Float16*>(a.packed + a.off_rnorm + vec * 2);
        } else {
#pragma unroll
            for (int k = 0; k < NW; ++k) w[k] = 0u;
        }
        half8 kb[KS];
        dequant_f16<C, B>(w, lut, kb);
        half8 sb[QJL ? KS : 1];
        if constexpr (QJL) {
            const uint8_t* sp = a.packed + a.off_sketch + vec * (int64_t)(m / 8) + g * (m / 32);
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const uint32_t byte = (valid && k < mks) ? sp[k] : 0u;
                sb[k] = *reinterpret_cast<const half8*>(sgn + byte * 8);
            }
        }
        const float c1 = n16, c2 = n16 * lam * r16;
        for (int qt = 0; qt < nqt; ++qt) {
            const int64_t qrow = st * a.n_q + qt * 16 + t16;   // A-operand row for this lane
            floatx4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
            const _Float16* qa = a.q_rot + qrow * D + g * C;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const half8 A = *reinterpret_cast<const half8*>(qa + 8 * k);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, kb[k], acc1, 0, 0, 0);
            }
            floatx4 acc2 = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (QJL) {
                const _Float16* pa = a.p + qrow * m + g * (m / 4);
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    if (k < mks) {
                        const half8 A = *reinterpret_cast<const half8*>(pa + 8 * k);
                        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, sb[k], acc2, 0, 0, 0);
                    }
                }
            }
            if (valid) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = qt * 16 + 4 * g + i;
                    if (q < a.n_q) {
                        const float sv = QJL ? fmaf(acc2[i], c2, acc1[i] * c1) : acc1[i] * c1;
                        a.scores[(st * a.n_q + q) * a.n_tokens + tok] = sv;
                    }
                }
            }
        }
    }
}

template <int D, int B, bool QJL>
static hipError_t launch_one(const ScoresArgs& a, int num_cus, hipStream_t s) {
    ScoresArgs b = a;
    const int64_t target = (int64_t)num_cus * 4;
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    hipLaunchKernelGGL((scores_kernel<D, B, QJL>), dim3((unsigned)(a.n_streams * bps)), dim3(256), 0, s, b);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const ScoresArgs& a, int num_cus, hipStream_t s) {
    const bool q = a.t.m > 0;
#define TQ_SC_CASE(BB) \
    case BB: return q ? launch_one<D, BB, true>(a, num_cus, s) : launch_one<D, BB, false>(a, num_cus, s);
    switch (a.t.b) {
        TQ_SC_CASE(1) TQ_SC_CASE(2) TQ_SC_CASE(3) TQ_SC_CASE(4)
        TQ_SC_CASE(5) TQ_SC_CASE(6) TQ_SC_CASE(7) TQ_SC_CASE(8)
    }
#undef TQ_SC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_scores(const ScoresArgs& a, int num_cus, hipStream_t s) {
    switch (a.t.d) {
        case 64: return launch_d<64>(a, num_cus, s);
        case 128: return launch_d<128>(a, num_cus, s);
        case 256: return launch_d<256>(a, num_cus, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
