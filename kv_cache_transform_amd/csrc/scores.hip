// Query preparation and score estimation on packed keys ("Ablation, Statistical Inference, and
// Validation for KV-Cache Compression", §2: TurboQuant paragraph — QJL on K improves the score
// estimate <q,k>; SpectralQuant paragraph — the asymmetric 1-bit estimator; here in the WHT domain
// with a Gaussian S):
//   q_rot = H (q ⊙ s) / sqrt(d),  p = S q_rot,
//   ŝ(q, k) = n16 · ( <q_rot, c[idx]> + sqrt(pi/2)/m · r16 · <p, 2σ - 1> ).
// The two contractions over d and m are v_mfma_f32_16x16x32_f16 tiles: A = 16 queries (fp16 hi + lo
// parts of q_rot / p), B = 16 keys dequantised straight from the packed bytes (hi + lo parts of the
// centroids, or the exact ±1 signs).  Lane l holds key l%16 and the
// k-block l/16, which is exactly the contiguous packed chunk g = l/16 the encoder wrote.
#include <map>
#include <mutex>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace tq {

// ---------------------------------------------------------------------------------------------
// q_rot and p per query row; one block of 256 threads per row (tiny amount of work, so the kernel is
// latency-bound: every load is issued up front).  Thread i < m fetches row i of S as D/8 16-byte
// pieces before anything else; the first wave loads the query, flips its signs and rotates it in
// registers (lane l holds coordinates (D/64) l + c: the low index bits in the lane, the rest as
// lane-xor butterflies, stage by stage from the lowest bit); then p_i = sum_j S_ij q_rot_j in
// index order.  Both are formed in fp32, scaled by the row's power of two 2^e (the largest |entry|
// of the two in [2^13, 2^14)) and written as fp16 hi + lo parts: hi the nearest fp16, lo the nearest
// fp16 of the remainder, so hi + lo is within ~2^-22 of the fp32 value for every entry above the
// fp16 subnormal range (2^-14 of a unit at most 2^-27 of the row's largest entry).
template <int D>
__global__ __launch_bounds__(256) void qprep_kernel(QPrepArgs a) {
    constexpr int PL = D / 64, NS = D / 8;
    const int64_t row = blockIdx.x;
    const int m = a.t.m, tid = threadIdx.x, lane = tid & 63;
    const int head = (int)((row / a.n_q_per_stream) % a.t.n_heads);
    __shared__ float buf[D], red[4];
    u32x4 srow[NS];
    if (tid < m) {
        const u32x4* sp = reinterpret_cast<const u32x4*>(a.t.S + ((int64_t)head * m + tid) * D);
#pragma unroll
        for (int k = 0; k < NS; ++k) srow[k] = sp[k];
    }
    const bool rot = a.t.rotation != 1;               // no rotation: q_rot = q
    if (tid < 64) {
        float v[PL];
        const float* sg = a.t.signs + (int64_t)head * D + PL * lane;
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
        for (int c = 0; c < PL; ++c) buf[PL * lane + c] = v[c];
    }
    __syncthreads();
    float mx = 0.0f, p = 0.0f;
    if (tid < m) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const half8 hs = __builtin_bit_cast(half8, srow[k]);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc = fmaf((float)hs[u], buf[8 * k + u], acc);
        }
        p = acc * a.p_scale;
        mx = fabsf(p);
    }
    if (tid < D) mx = fmaxf(mx, fabsf(buf[tid] * a.q_scale));
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // 2^e with the row's largest entry in [2^13, 2^14); an all-zero (or non-finite) row keeps e = 0
    const int ex = (int)((f2u(mx) >> 23) & 0xffu);
    const int e = (mx > 0.0f && ex < 255) ? 13 - (ex == 0 ? -126 : ex - 127) : 0;
    auto split = [&](float v, _Float16* hp, _Float16* lp, int64_t k) {
        const float sv = __builtin_amdgcn_ldexpf(v, e);
        const _Float16 h = (_Float16)sv;
        hp[k] = h;
        lp[k] = (_Float16)(sv - (float)h);
    };
    if (tid < D) split(buf[tid] * a.q_scale, a.o.qh, a.o.ql, row * D + tid);
    if (tid < m) split(p, a.o.ph, a.o.pl, row * m + tid);
    if (tid == 0) a.o.rowf[row] = __builtin_amdgcn_ldexpf(1.0f, -e);
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s) {
    if (a.n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)a.n_rows);
    switch (a.t.d) {
        case 64: hipLaunchKernelGGL(qprep_kernel<64>, grid, dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL(qprep_kernel<128>, grid, dim3(256), 0, s, a); break;
        case 256: hipLaunchKernelGGL(qprep_kernel<256>, grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Dequantise the lane's C packed coordinates into C/8 pairs of fp16x8 MFMA operands: hi and lo parts
// of 2^12 c[idx] (the LUT entry of P coordinates holds their P hi parts, then their P lo parts).
template <int C, int B>
__device__ __forceinline__ void dequant_hl(const uint32_t (&w)[(C * B + 31) / 32], const _Float16* lut,
                                           half8 (&oh)[C / 8], half8 (&ol)[C / 8]) {
    constexpr int P = lut_group_c(B);
#pragma unroll
    for (int k = 0; k < C / 8; ++k) {
        if constexpr (P == 8) {
            const uint32_t f = get_bits<8 * B>(w, (8 * k) * B);
            oh[k] = *reinterpret_cast<const half8*>(lut + f * 16);
            ol[k] = *reinterpret_cast<const half8*>(lut + f * 16 + 8);
        } else if constexpr (P == 4) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t f = get_bits<4 * B>(w, (8 * k + 4 * h) * B);
                const half8 e = *reinterpret_cast<const half8*>(lut + f * 8);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    oh[k][4 * h + u] = e[u];
                    ol[k][4 * h + u] = e[4 + u];
                }
            }
        } else if constexpr (P == 2) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t f = get_bits<2 * B>(w, (8 * k + 2 * h) * B);
                const half4 e = *reinterpret_cast<const half4*>(lut + f * 4);
                oh[k][2 * h] = e[0];
                oh[k][2 * h + 1] = e[1];
                ol[k][2 * h] = e[2];
                ol[k][2 * h + 1] = e[3];
            }
        } else {
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const uint32_t f = get_bits<B>(w, (8 * k + h) * B);
                const half2v e = *reinterpret_cast<const half2v*>(lut + f * 2);
                oh[k][h] = e[0];
                ol[k][h] = e[1];
            }
        }
    }
}

// Scores of 16 keys (one wave tile) against all queries of the stream.  Lane (t16, g) holds key
// t16's packed chunk g (its B-operand rows), dequantised through an LDS LUT into fp16 hi + lo parts
// of 2^12 c; the queries (hi + lo parts of 2^e q_rot, and of 2^e S q_rot with the sketch) are A
// operands, staged once per block in LDS (rows padded by 16 bytes so a 16-lane column read spreads
// over the banks) when they fit, else read from the workspace.  <q_rot, c> takes the three products
// hi·hi + lo·hi + hi·lo and <p, 2σ - 1> the two products with the exact ±1 signs, so only the fp32
// accumulation rounds: the scores are fp32-accurate, also for a short row or a cancelling score.
// The next tile's packed bytes, norms and sketch words are loaded while the current tile is
// computed.  Output lane (t16, g) holds queries 4g + i of key t16: each store writes, per query, 16
// consecutive keys.
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
    constexpr int LUT_B = (NE * P * 4 + 15) & ~15;
    u32x2* sgn4 = reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(smem4) + LUT_B);
    uint8_t* qbase = reinterpret_cast<uint8_t*>(smem4) + LUT_B + 128;
    const int m = a.t.m;
    const int nqp = (a.n_q + 15) & ~15;          // staged rows (zero past n_q)
    constexpr int QSD = D + 8;                   // padded row of staged queries (halves)
    const int QSM = m + 8;                       // padded row of staged projections
    float* rfs = reinterpret_cast<float*>(qbase);                   // [nqp] row factors
    _Float16* qsh = reinterpret_cast<_Float16*>(qbase + nqp * 4);
    _Float16* qsl = qsh + nqp * QSD;
    _Float16* psh = qsl + nqp * QSD;
    _Float16* psl = psh + nqp * QSM;

    const int64_t st = blockIdx.x / a.blocks_per_stream;
    for (int i = threadIdx.x; i < NE * P * 2; i += blockDim.x) lut[i] = a.t.lut_hl[i];
    if (threadIdx.x < 16) {
        uint32_t w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            w[j] = (((threadIdx.x >> (2 * j)) & 1) ? 0x3c00u : 0xbc00u) |
                   ((((threadIdx.x >> (2 * j + 1)) & 1) ? 0x3c00u : 0xbc00u) << 16);
        sgn4[threadIdx.x] = u32x2{w[0], w[1]};
    }
    if constexpr (QL) {
        // stage this stream's query operands: 8 halves (16 bytes) per thread step
        for (int i = threadIdx.x; i < nqp; i += blockDim.x) rfs[i] = i < a.n_q ? a.o.rowf[st * a.n_q + i] : 0.0f;
        for (int i = threadIdx.x; i < nqp * (D / 8); i += blockDim.x) {
            const int r = i / (D / 8), c8 = i - r * (D / 8);
            u32x4 vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
            if (r < a.n_q) {
                vh = *reinterpret_cast<const u32x4*>(a.o.qh + (st * a.n_q + r) * D + 8 * c8);
                vl = *reinterpret_cast<const u32x4*>(a.o.ql + (st * a.n_q + r) * D + 8 * c8);
            }
            *reinterpret_cast<u32x4*>(qsh + r * QSD + 8 * c8) = vh;
            *reinterpret_cast<u32x4*>(qsl + r * QSD + 8 * c8) = vl;
        }
        if constexpr (QJL)
            for (int i = threadIdx.x; i < nqp * (m / 8); i += blockDim.x) {
                const int r = i / (m / 8), c8 = i - r * (m / 8);
                u32x4 vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
                if (r < a.n_q) {
                    vh = *reinterpret_cast<const u32x4*>(a.o.ph + (st * a.n_q + r) * m + 8 * c8);
                    vl = *reinterpret_cast<const u32x4*>(a.o.pl + (st * a.n_q + r) * m + 8 * c8);
                }
                *reinterpret_cast<u32x4*>(psh + r * QSM + 8 * c8) = vh;
                *reinterpret_cast<u32x4*>(psl + r * QSM + 8 * c8) = vl;
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
        half8 kh[KS], kl[KS];
        dequant_hl<C, B>(cur.w, lut, kh, kl);
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
        const float c1 = n16 * (1.0f / 4096.0f);           // undoes the 2^12 of the centroid parts
        const float c2 = QJL ? n16 * lam * (float)__builtin_bit_cast(_Float16, cur.r16) : 0.0f;
        float* orow = a.scores + (st * a.n_q) * a.n_tokens + tok;
        for (int qt = 0; qt < nqt; ++qt) {
            const int qr = qt * 16 + t16;                    // A-operand row for this lane
            floatx4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int64_t go = (st * a.n_q + qr) * D + g * C + 8 * k;
                const half8 Ah = QL ? *reinterpret_cast<const half8*>(qsh + qr * QSD + g * C + 8 * k)
                                    : *reinterpret_cast<const half8*>(a.o.qh + go);
                const half8 Al = QL ? *reinterpret_cast<const half8*>(qsl + qr * QSD + g * C + 8 * k)
                                    : *reinterpret_cast<const half8*>(a.o.ql + go);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, kh[k], acc1, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, kh[k], acc1, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, kl[k], acc1, 0, 0, 0);
            }
            floatx4 acc2 = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (QJL) {
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    if (k < mks) {
                        const int64_t go = (st * a.n_q + qr) * m + g * (m / 4) + 8 * k;
                        const half8 Ah = QL ? *reinterpret_cast<const half8*>(psh + qr * QSM + g * (m / 4) + 8 * k)
                                            : *reinterpret_cast<const half8*>(a.o.ph + go);
                        const half8 Al = QL ? *reinterpret_cast<const half8*>(psl + qr * QSM + g * (m / 4) + 8 * k)
                                            : *reinterpret_cast<const half8*>(a.o.pl + go);
                        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, sb[k], acc2, 0, 0, 0);
                        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, sb[k], acc2, 0, 0, 0);
                    }
                }
            }
            if (valid) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = qt * 16 + 4 * g + i;
                    if (q < a.n_q) {
                        const float rf = QL ? rfs[q] : a.o.rowf[st * a.n_q + q];
                        const float v = QJL ? fmaf(acc2[i], c2, acc1[i] * c1) : acc1[i] * c1;
                        orow[(int64_t)q * a.n_tokens] = v * rf;
                    }
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
    const size_t lut_b = (size_t)((NE * P * 4 + 15) & ~15) + 128;
    const int nqp = (a.n_q + 15) & ~15;
    const size_t q_b = (size_t)nqp * 4 + (size_t)nqp * (D + 8) * 4 + (QJL ? (size_t)nqp * (a.t.m + 8) * 4 : 0);
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
