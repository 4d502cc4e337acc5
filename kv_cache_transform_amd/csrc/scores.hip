// Query preparation and score estimation on packed keys ("Ablation, Statistical Inference, and
// Validation for KV-Cache Compression", §2: TurboQuant paragraph — QJL on K improves the score
// estimate <q,k>; SpectralQuant paragraph — the asymmetric 1-bit estimator; here in the WHT domain
// with a Gaussian S):
//   q_rot = H (q ⊙ s) / sqrt(d),  p = S q_rot,
//   ŝ(q, k) = n16 · ( <q_rot, c[idx]> + sqrt(pi/2)/m · r16 · <p, 2σ - 1> ).
// The two contractions over d and m are v_mfma_f32_16x16x32_f16 tiles: A = 16 queries (fp16
// q_rot / p), B = 16 keys dequantised straight from the packed bytes.  Lane l holds key l%16 and the
// k-block l/16, which is exactly the contiguous packed chunk g = l/16 the encoder wrote.
#include <map>
#include <mutex>
#include <utility>

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
        buf[j] = a.t.rotation == 1 ? x : x * sg[j];
    }
    __syncthreads();
    for (int h = 1; h < (a.t.rotation == 1 ? 1 : d); h <<= 1) {   // no rotation: q_rot = q
        for (int i = threadIdx.x; i < d / 2; i += blockDim.x) {
            const int lo = (i / h) * 2 * h + (i % h);
            const float x0 = buf[lo], x1 = buf[lo + h];
            buf[lo] = x0 + x1;
            buf[lo + h] = x0 - x1;
        }
        __syncthreads();
    }
    const float inv = a.t.rotation == 1 ? 1.0f : 1.0f / sqrtf((float)d);
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

// Scores of 16 keys (one wave tile) against all queries of the stream.  Lane (t16, g) holds key
// t16's packed chunk g (its B-operand rows), dequantised to fp16 through an LDS LUT; the queries
// (q_rot, and p = S q_rot with the sketch) are A operands, staged once per block in LDS (rows padded
// by 16 bytes so a 16-lane column read spreads over the banks) when they fit, else read from the
// workspace.  The next tile's packed bytes, norms and sketch words are loaded while the current
// tile is computed.  Output lane (t16, g) holds queries 4g + i of key t16: each store writes, per
// query, 16 consecutive keys.
template <int D, int B, bool QJL, bool QL>
__global__ __launch_bounds__(256) void scores_kernel(ScoresArgs a) {
    constexpr int C = D / 4;
    constexpr int P = lut_group_c(B), NE = 1 << (P * B);
    constexpr int NW = (C * B + 31) / 32;
    constexpr int CB = C * B / 8;
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr int KS = C / 8;                   // k-steps over d (and the maximum over m <= d)
    constexpr int NKS = D >= 256 ? 2 : 1;       // sketch words per lane (m/32 bytes <= 8)

    extern __shared__ uint4 smem4[];
    _Float16* lut = reinterpret_cast<_Float16*>(smem4);
    constexpr int LUT_B = (NE * P * 2 + 15) & ~15;
    u32x2* sgn4 = reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(smem4) + LUT_B);
    _Float16* qs = reinterpret_cast<_Float16*>(reinterpret_cast<uint8_t*>(smem4) + LUT_B + 128);
    const int m = a.t.m;
    const int nqp = (a.n_q + 15) & ~15;          // staged rows (zero past n_q)
    constexpr int QSD = D + 8;                   // padded row of staged q_rot (halves)
    const int QSM = m + 8;                       // padded row of staged p
    _Float16* ps = qs + nqp * QSD;

    const int64_t st = blockIdx.x / a.blocks_per_stream;
    for (int i = threadIdx.x; i < NE * P; i += blockDim.x) lut[i] = a.t.lut_f16[i];
    if (threadIdx.x < 16) {
        uint32_t w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            w[j] = (((threadIdx.x >> (2 * j)) & 1) ? 0x3c00u : 0xbc00u) |
                   ((((threadIdx.x >> (2 * j + 1)) & 1) ? 0x3c00u : 0xbc00u) << 16);
        sgn4[threadIdx.x] = u32x2{w[0], w[1]};
    }
    if constexpr (QL) {
        // stage this stream's queries: 8 halves (16 bytes) per thread step
        for (int i = threadIdx.x; i < nqp * (D / 8); i += blockDim.x) {
            const int r = i / (D / 8), c8 = i - r * (D / 8);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < a.n_q) v = *reinterpret_cast<const u32x4*>(a.q_rot + (st * a.n_q + r) * D + 8 * c8);
            *reinterpret_cast<u32x4*>(qs + r * QSD + 8 * c8) = v;
        }
        if constexpr (QJL)
            for (int i = threadIdx.x; i < nqp * (m / 8); i += blockDim.x) {
                const int r = i / (m / 8), c8 = i - r * (m / 8);
                u32x4 v = {0u, 0u, 0u, 0u};
                if (r < a.n_q) v = *reinterpret_cast<const u32x4*>(a.p + (st * a.n_q + r) * m + 8 * c8);
                *reinterpret_cast<u32x4*>(ps + r * QSM + 8 * c8) = v;
            }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int t16 = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int mks = m >> 5;                     // sketch k-steps (m/4 bits per lane, 8 per step)
    const float lam = QJL ? 1.2533141373155003f / (float)m : 0.0f;   // sqrt(pi/2)/m
    const int nqt = (a.n_q + 15) >> 4;
    const uint32_t ksh = (uint32_t)((g * (m >> 5)) & 3) * 8u;       // bit offset of the sketch bytes

    // packed bytes, norms and sketch words of one tile (a key past the end reads key 0 of the
    // stream: in bounds, never stored)
    struct Tile {
        uint32_t w[NW];
        uint32_t ks[NKS + 1];
        uint16_t n16, r16;
    };
    auto load_tile = [&](Tile& T, int64_t tile) {
        const int64_t tok = tile * 16 + t16;
        const int64_t vec = st * a.n_tokens + (tok < a.n_tokens ? tok : 0);
        load_bytes<CB, CA>(a.packed + a.off_idx + vec * (int64_t)(D * B / 8) + g * CB, T.w);
        T.n16 = *reinterpret_cast<const uint16_t*>(a.packed + a.off_norm + vec * 2);
        if constexpr (QJL) {
            T.r16 = *reinterpret_cast<const uint16_t*>(a.packed + a.off_rnorm + vec * 2);
            const uint8_t* sp = a.packed + a.off_sketch + vec * (int64_t)(m / 8) + ((g * (m / 32)) & ~3);
#pragma unroll
            for (int k = 0; k <= NKS; ++k) T.ks[k] = reinterpret_cast<const uint32_t*>(sp)[k];
        }
    };
    Tile nx;
    if (tb0 + wave < tb1) load_tile(nx, tb0 + wave);

#pragma unroll 1
    for (int64_t tile = tb0 + wave; tile < tb1; tile += 4) {
        const Tile cur = nx;
        if (tile + 4 < tb1) load_tile(nx, tile + 4);     // next tile's loads overlap this tile
        const int64_t tok = tile * 16 + t16;
        const bool valid = tok < a.n_tokens;
        half8 kb[KS];
        dequant_f16<C, B>(cur.w, lut, kb);
        half8 sb[QJL ? KS : 1];
        if constexpr (QJL) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const uint32_t wsk = __builtin_amdgcn_alignbit(cur.ks[(k >> 2) + 1], cur.ks[k >> 2], ksh);
                const uint32_t byte = (wsk >> (8 * (k & 3))) & 0xffu;
                const u32x2 lo = sgn4[byte & 0xfu], hi = sgn4[byte >> 4];
                sb[k] = __builtin_bit_cast(half8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        }
        const float n16 = (float)__builtin_bit_cast(_Float16, cur.n16);
        const float c1 = n16, c2 = QJL ? n16 * lam * (float)__builtin_bit_cast(_Float16, cur.r16) : 0.0f;
        float* orow = a.scores + (st * a.n_q) * a.n_tokens + tok;
        for (int qt = 0; qt < nqt; ++qt) {
            const int qr = qt * 16 + t16;                    // A-operand row for this lane
            floatx4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const half8 A = QL ? *reinterpret_cast<const half8*>(qs + qr * QSD + g * C + 8 * k)
                                   : *reinterpret_cast<const half8*>(a.q_rot + (st * a.n_q + qr) * D + g * C + 8 * k);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, kb[k], acc1, 0, 0, 0);
            }
            floatx4 acc2 = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (QJL) {
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    if (k < mks) {
                        const half8 A = QL ? *reinterpret_cast<const half8*>(ps + qr * QSM + g * (m / 4) + 8 * k)
                                           : *reinterpret_cast<const half8*>(a.p + (st * a.n_q + qr) * m + g * (m / 4) + 8 * k);
                        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, sb[k], acc2, 0, 0, 0);
                    }
                }
            }
            if (valid) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = qt * 16 + 4 * g + i;
                    if (q < a.n_q) orow[(int64_t)q * a.n_tokens] = QJL ? fmaf(acc2[i], c2, acc1[i] * c1) : acc1[i] * c1;
                }
            }
        }
    }
}

// resident blocks per CU of kernel k at `lds` bytes of dynamic LDS (cached per kernel and size)
static int scores_blocks_per_cu(const void* k, size_t lds) {
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

template <int D, int B, bool QJL>
static hipError_t launch_one(const ScoresArgs& a, int num_cus, hipStream_t s) {
    ScoresArgs b = a;
    constexpr int P = lut_group_c(B), NE = 1 << (P * B);
    const size_t lut_b = (size_t)((NE * P * 2 + 15) & ~15) + 128;
    const int nqp = (a.n_q + 15) & ~15;
    const size_t q_b = (size_t)nqp * (D + 8) * 2 + (QJL ? (size_t)nqp * (a.t.m + 8) * 2 : 0);
    const bool ql = lut_b + q_b <= 98304;        // stage the queries when they fit in 96 KiB
    const size_t lds = lut_b + (ql ? q_b : 0);
    const void* kern = ql ? reinterpret_cast<const void*>(&scores_kernel<D, B, QJL, true>)
                          : reinterpret_cast<const void*>(&scores_kernel<D, B, QJL, false>);
    const int64_t target = (int64_t)num_cus * scores_blocks_per_cu(kern, lds);
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    const dim3 grid((unsigned)(a.n_streams * bps));
    if (ql) hipLaunchKernelGGL((scores_kernel<D, B, QJL, true>), grid, dim3(256), lds, s, b);
    else hipLaunchKernelGGL((scores_kernel<D, B, QJL, false>), grid, dim3(256), lds, s, b);
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
