// SpectralQuant kernels for gfx950: projection onto a calibrated eigenbasis with per-dimension
// Gaussian Lloyd-Max codebooks and variable-width records ("Ablation, Statistical Inference, and
// Validation for KV-Cache Compression", §2 "SpectralQuant": z = Uᵀk, the semantic dimensions at
// their water-filled widths and the tail at b_tail bits; the score <Uᵀq, ẑ>).
//
// MFMA layout (v_mfma_f32_16x16x32_f16): lane l supplies A[l%16][8(l/16)+i] and B[8(l/16)+i][l%16],
// i = 0..7, and receives D[4(l/16)+r][l%16], r = 0..3.  A wave works on 16 vectors at a time.
//
//   encode  D[vector][k] = Σ_j x[vector][j] · Uᵀ[j][k]: A = the vectors (bf16 scaled by a power of
//           two per vector into fp16, exactly), B = U·2^8 as an fp16 hi + lo pair from LDS, two
//           products per step.  Lane (n = l%16, g) ends with coordinate k = 16t + n of vectors
//           4g + r, so its per-dimension constants (scale, grid, bit offset, width) stay in
//           registers.  The 4 lanes of a quad hold dimensions 4q..4q+3, whose fields are adjacent:
//           their shifted indices are OR-ed together over DPP, the quad's first lane ORs the group
//           into the vector's record in LDS (ds_or), and the wave's 16 records are then written
//           out linearly.
//   decode  D[j][vector] = Σ_k (U diag σ)[j][k] · c[vector][k]: A = U diag(σ)·2^e as hi + lo from LDS,
//           B = the codebook values as hi + lo of c·2^12 (three products per step, about 2^-21
//           relative).  Lane (v, g) extracts its 8 contiguous fields k = 32s + 8g + i of vector v
//           per step from the record staged in LDS.
//   scores  D[query][token] = Σ_k (q_Z ⊙ σ)[query][k] · c[token][k] with fp16 operands, the query side
//           projected once per row by `sq_qprep_kernel`.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "common.hpp"
#include "sq_kernels.hpp"

namespace tq {

namespace {

constexpr size_t kLdsMax = 163840;

__device__ __forceinline__ half8 as_half8(const u32x4& w) { return __builtin_bit_cast(half8, w); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// OR of v over the 4 lanes of its quad (DPP quad permutations [1,0,3,2] then [2,3,0,1])
__device__ __forceinline__ uint32_t quad_or(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, true);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, true);
    return v;
}

// bf16 pair (one word) times 2^sc into an fp16 pair (exact for every value within 2^-24 of the
// vector's largest; smaller ones are truncated to the fp16 subnormal grid)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_scaled(uint32_t w, int sc) {
    const float f0 = __builtin_amdgcn_ldexpf(u2f(w << 16), sc);
    const float f1 = __builtin_amdgcn_ldexpf(u2f(w & 0xffff0000u), sc);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1));
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// records of `count` words starting at `src` (valid words < n_valid) into registers, one word per
// lane per step; NP steps cover up to 64·NP words
template <int NP>
__device__ __forceinline__ void fetch_words(const uint32_t* src, int count, int n_valid, int lane, uint32_t (&w)[NP]) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int i = lane + 64 * j;
        w[j] = (i < count && i < n_valid) ? src[i] : 0u;
    }
}

// `width` (1..31) bits from bit `pos` of a record in LDS (reads the word after the one holding pos)
__device__ __forceinline__ uint32_t get_bits_at(const uint32_t* rec, uint32_t pos, uint32_t width) {
    const uint32_t* w = rec + (pos >> 5);
    return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[1], w[0], pos & 31u), 0, width);
}

// the lane's 8 fields of one k-step: the 64 bits from bit r0 of record word w0 hold them all; each
// comes out as its row index width·256 + value of the [width][256] codebook tables
__device__ __forceinline__ void fields8(const uint32_t* rec, const uint4& fd, uint32_t (&ix)[8]) {
    const uint32_t* w = rec + (fd.x & 0xffu);
    const uint32_t r0 = fd.x >> 8;
    const uint32_t d0 = w[0], d1 = w[1], d2 = w[2];
    const uint64_t win = ((uint64_t)__builtin_amdgcn_alignbit(d2, d1, r0) << 32) | __builtin_amdgcn_alignbit(d1, d0, r0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t pos = i == 0 ? 0u : __builtin_amdgcn_ubfe(i <= 4 ? fd.y : fd.z, 8 * ((i - 1) & 3), 8);
        const uint32_t wid = __builtin_amdgcn_ubfe(fd.w, 4 * i, 4);
        ix[i] = (wid << 8) | __builtin_amdgcn_ubfe((uint32_t)(win >> pos), 0, wid);
    }
}

int blocks_per_cu(const void* k, int threads, size_t lds) {
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

hipError_t raise_lds(const void* kern) {
    static std::mutex mu;
    static std::map<const void*, bool> done;
    std::lock_guard<std::mutex> lock(mu);
    if (done[kern]) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (e == hipSuccess) done[kern] = true;
    return e;
}

template <typename Args>
void split_grid(Args& b, const void* kern, int threads, size_t lds, int num_cus) {
    const int64_t target = (int64_t)num_cus * blocks_per_cu(kern, threads, lds);
    int64_t bps = (target + b.n_streams - 1) / b.n_streams;
    if (bps > b.tiles_per_stream) bps = b.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (b.tiles_per_stream + bps - 1) / bps;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------------------------
constexpr int kEncThreads = 512;

// SK: the codec carries the selective sketch (compiled apart so that the plain path keeps its registers)
template <int D, int NG, bool SK>
__global__ __launch_bounds__(kEncThreads, 1) void sq_encode_kernel(SqEncodeArgs a) {
    constexpr int T = D / 16, S = D / 32;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kEncThreads / 64;
    const int n = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int RW = a.t.rec_words;
    u32x4* Bt = reinterpret_cast<u32x4*>(smem);                                 // [part][t][s][lane]
    uint2* grid = reinterpret_cast<uint2*>(smem + (size_t)2 * T * S * 1024);
    // per wave: 16 records and one pad word (the second word of a group at the end of the last record)
    const int WS = 16 * RW + 1;
    uint32_t* stage = reinterpret_cast<uint32_t*>(smem + (size_t)2 * T * S * 1024 +
                                                  (size_t)((a.t.lds_grid_words + 3) / 4) * 16) +
                      wave * WS;
    // with the selective sketch: after all waves' records, a 16 x 32-word transposition buffer per
    // wave, then the ±1 sketch tiles of this head
    const int M = SK ? a.t.m : 0;
    uint32_t* tbuf = reinterpret_cast<uint32_t*>(smem + (size_t)2 * T * S * 1024 +
                                                 (size_t)((a.t.lds_grid_words + 3) / 4) * 16) +
                     (kEncThreads / 64) * WS + wave * 512;
    u32x4* skt = reinterpret_cast<u32x4*>(reinterpret_cast<uint32_t*>(smem + (size_t)2 * T * S * 1024 +
                                                                      (size_t)((a.t.lds_grid_words + 3) / 4) * 16) +
                                          (kEncThreads / 64) * (WS + 512));
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.enc_b) + (size_t)head * 2 * T * S * 64;
        for (int i = threadIdx.x; i < 2 * T * S * 64; i += kEncThreads) Bt[i] = src[i];
        uint32_t* gw = reinterpret_cast<uint32_t*>(grid);
        for (int i = threadIdx.x; i < a.t.lds_grid_words; i += kEncThreads) gw[i] = a.t.grids[i];
        for (int i = lane; i < WS; i += 64) stage[i] = 0u;
        if (M > 0) {
            const u32x4* ks = reinterpret_cast<const u32x4*>(a.t.sk_b) + (size_t)head * (M / 16) * 64;
            for (int i = threadIdx.x; i < (M / 16) * 64; i += kEncThreads) skt[i] = ks[i];
        }
    }
    const int deff = M > 0 ? a.t.deff[head] : 0;
    const uint32_t skoff = M > 0 ? (uint32_t)a.t.sk_off[head] : 0u;
    float sgk[2] = {0.0f, 0.0f};
    if (M > 0) {
        sgk[0] = a.t.sigma[(size_t)head * D + n];
        sgk[1] = a.t.sigma[(size_t)head * D + 16 + n];
    }
    float mul[T], add[T];
    uint32_t meta[T], meta2[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float4 dsc = a.t.enc_desc[(size_t)head * D + 16 * t + n];
        mul[t] = dsc.x;
        add[t] = dsc.y;
        meta[t] = f2u(dsc.z);
        meta2[t] = f2u(dsc.w);
    }
    __syncthreads();

    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint16_t* xs = a.x + (size_t)st * a.n_tokens * D;
    uint32_t* os = a.out + (size_t)st * a.n_tokens * RW;

    auto load = [&](int64_t tile, u32x4 (&raw)[S]) {
        const int64_t tok = tile * 16 + n;
        if (tile < t_end && tok < a.n_tokens) {
#pragma unroll
            for (int s = 0; s < S; ++s)
                raw[s] = *reinterpret_cast<const u32x4*>(xs + (size_t)tok * D + 32 * s + 8 * g);
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s) raw[s] = u32x4{0u, 0u, 0u, 0u};
        }
    };

    u32x4 raw[NG][S];
    int64_t tile = t_begin + (int64_t)wave * NG;
#pragma unroll
    for (int q = 0; q < NG; ++q) load(tile + q, raw[q]);
    for (; tile < t_end; tile += (int64_t)nwaves * NG) {
        // per-vector power-of-two scale: the largest bf16 exponent of the vector (over its 4 lanes)
        half8 A[NG][S];
        int sc[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            // magnitudes as unsigned 16-bit pairs (monotone in |x|), maximum per half, then per lane
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, raw[q][s][w] & 0x7fff7fffu));
            uint32_t e2 = (uint32_t)max(m2[0], m2[1]) & 0x7f80u;
            uint32_t ea = e2, eb = e2;
            xswap16u(ea, eb);
            e2 = max(ea, eb);
            ea = e2;
            eb = e2;
            xswap32u(ea, eb);
            const int E = (int)(max(ea, eb) >> 7);
            sc[q] = E == 0 ? 0 : 141 - E;   // largest |x|·2^sc in [2^14, 2^15)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                u32x4 h;
#pragma unroll
                for (int w = 0; w < 4; ++w) h[w] = bf16x2_to_f16x2_scaled(raw[q][s][w], sc[q]);
                A[q][s] = as_half8(h);
            }
        }
        const int64_t next = tile + (int64_t)nwaves * NG;
#pragma unroll
        for (int q = 0; q < NG; ++q) load(next + q, raw[q]);

        floatx4 acc[NG][T];
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[q][t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const half8 bh = as_half8(Bt[(t * S + s) * 64 + lane]);
                const half8 bl = as_half8(Bt[((T + t) * S + s) * 64 + lane]);
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[q][s], bh, acc[q][t], 0, 0, 0);
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[q][s], bl, acc[q][t], 0, 0, 0);
                }
            }

#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t tq_ = tile + q;
            if (tq_ >= t_end) break;
            int scr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) scr[r] = __shfl(sc[q], 4 * g + r);
            uint32_t ik[2][4];   // the indices of dimensions n and 16 + n (the sketch's residual)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t goff = meta[t] & 0xffffu, qrel = meta2[t] & 0xffu;
                uint32_t val[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float z = __builtin_amdgcn_ldexpf(acc[q][t][r], -scr[r]);
                    const float ug = fmaf(z, mul[t], add[t]);
                    const int cell = (int)__builtin_amdgcn_fmed3f(ug, 0.0f, 2.0f * add[t]);
                    const uint2 e = grid[goff + cell];
                    const uint32_t ix = e.y + (ug >= u2f(e.x) ? 1u : 0u);
                    if (t < 2) ik[t][r] = ix;
                    // the 4 neighbouring dimensions 4q..4q+3 (the lanes of one quad) OR-ed together
                    val[r] = quad_or(ix << qrel);
                }
                // the quad's first lane ORs the group's bits into its record (two words; the second
                // is zero unless the group straddles them)
                if ((lane & 3) == 0) {
                    const uint32_t off = (meta[t] >> 16) & 0x3ffu, wi = off >> 5, sh = off & 31u;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint64_t v64 = (uint64_t)val[r] << sh;
                        uint32_t* rec = stage + (4 * g + r) * RW + wi;
                        atomicOr(rec, (uint32_t)v64);
                        atomicOr(rec + 1, (uint32_t)(v64 >> 32));
                    }
                }

            }
            if (M > 0) {
                // selective QJL sketch: e = z - σ c[idx] on the semantic dimensions (all among the
                // first 32, which lanes n hold in tiles 0 and 1), its norm over the 16-lane row, then
                // S e on MFMA after a transposition through LDS into the vectors' operand layout
                float ev[2][4], r2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint32_t wid = meta[t] >> 26;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float z = __builtin_amdgcn_ldexpf(acc[q][t][r], -(8 + scr[r]));
                        const float c = a.t.cent32[(wid << 8) | ik[t][r]];
                        const float e = (16 * t + n < deff) ? fmaf(-sgk[t], c, z) : 0.0f;
                        ev[t][r] = e;
                        r2[r] = fmaf(e, e, r2[r]);
                    }
                }
                float nrm[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = r2[r];
                    v += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0xb1, 0xf, 0xf, false));
                    v += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x4e, 0xf, 0xf, false));
                    v += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x141, 0xf, 0xf, false));
                    v += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x140, 0xf, 0xf, false));
                    nrm[r] = sqrtf(v);
                    const int es = nrm[r] > 0.0f ? 141 - (int)((f2u(nrm[r]) >> 23) & 0xffu) : 0;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const float x = __builtin_amdgcn_ldexpf(ev[t][r], es);
                        const _Float16 hi = (_Float16)x, lo = (_Float16)(x - (float)hi);
                        tbuf[(4 * g + r) * 32 + 16 * t + n] =
                            (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
                    }
                }
                // operand layout: lane (n, g) takes dimensions 8g..8g+7 of vector n
                const u32x4 w0 = reinterpret_cast<const u32x4*>(tbuf)[(n * 32 + 8 * g) / 4];
                const u32x4 w1 = reinterpret_cast<const u32x4*>(tbuf)[(n * 32 + 8 * g) / 4 + 1];
                u32x4 hv, lv;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    hv[i] = __builtin_amdgcn_perm(w0[2 * i + 1], w0[2 * i], 0x05040100u);
                    lv[i] = __builtin_amdgcn_perm(w0[2 * i + 1], w0[2 * i], 0x07060302u);
                    hv[2 + i] = __builtin_amdgcn_perm(w1[2 * i + 1], w1[2 * i], 0x05040100u);
                    lv[2 + i] = __builtin_amdgcn_perm(w1[2 * i + 1], w1[2 * i], 0x07060302u);
                }
                for (int ts = 0; ts < M / 16; ++ts) {
                    const half8 sb = as_half8(skt[ts * 64 + lane]);
                    floatx4 zs = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(hv), sb, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    zs = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(lv), sb, zs, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint64_t mask = __ballot(zs[r] >= 0.0f);   // lane (row n, g) -> bit 16g + n
                        if (n == 0) {
                            const uint32_t bits16 = (uint32_t)(mask >> (16 * g)) & 0xffffu;
                            const uint32_t pos = skoff + 16u * ts;
                            const uint64_t v64 = (uint64_t)bits16 << (pos & 31u);
                            uint32_t* rec = stage + (4 * g + r) * RW + (pos >> 5);
                            atomicOr(rec, (uint32_t)v64);
                            atomicOr(rec + 1, (uint32_t)(v64 >> 32));
                        }
                    }
                }
                if (n == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)nrm[r]);
                        const uint32_t pos = skoff + (uint32_t)M;
                        const uint64_t v64 = (uint64_t)h << (pos & 31u);
                        uint32_t* rec = stage + (4 * g + r) * RW + (pos >> 5);
                        atomicOr(rec, (uint32_t)v64);
                        atomicOr(rec + 1, (uint32_t)(v64 >> 32));
                    }
                }
            }
            // the wave's 16 records, written out linearly and the staging cleared
            const int64_t valid = min((int64_t)16, a.n_tokens - tq_ * 16);
            uint32_t* dst = os + (size_t)tq_ * 16 * RW;
            for (int i = lane; i < 16 * RW; i += 64) {
                const uint32_t v = stage[i];
                stage[i] = 0u;
                if (i < valid * RW) dst[i] = v;
            }
        }
    }
}

template <int D, bool SK>
static hipError_t launch_enc(const SqEncodeArgs& a, int num_cus, hipStream_t s) {
    constexpr int NG = 2;
    SqEncodeArgs b = a;
    const size_t lds = (size_t)2 * (D / 16) * (D / 32) * 1024 + (size_t)((a.t.lds_grid_words + 3) / 4) * 16 +
                       (size_t)(kEncThreads / 64) * (16 * a.t.rec_words + 1) * 4 +
                       (a.t.m > 0 ? (size_t)(kEncThreads / 64) * 512 * 4 + (size_t)(a.t.m / 16) * 1024 : 0);
    if (lds > kLdsMax) return hipErrorInvalidValue;
    const void* kern = reinterpret_cast<const void*>(&sq_encode_kernel<D, NG, SK>);
    if (lds > 65536) {
        const hipError_t e = raise_lds(kern);
        if (e != hipSuccess) return e;
    }
    split_grid(b, kern, kEncThreads, lds, num_cus);
    hipLaunchKernelGGL((sq_encode_kernel<D, NG, SK>), dim3((unsigned)(b.n_streams * b.blocks_per_stream)),
                       dim3(kEncThreads), lds, s, b);
    return hipGetLastError();
}

hipError_t launch_sq_encode(const SqEncodeArgs& a, int num_cus, hipStream_t s) {
    if (a.t.m > 0) return a.t.d == 64 ? launch_enc<64, true>(a, num_cus, s) : launch_enc<128, true>(a, num_cus, s);
    return a.t.d == 64 ? launch_enc<64, false>(a, num_cus, s) : launch_enc<128, false>(a, num_cus, s);
}

// ---------------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------------
constexpr int kDecThreads = 512;
constexpr int kCbRows = 9;   // codebook rows of widths 0..8

template <int D, bool BF, int NG>
__global__ __launch_bounds__(kDecThreads, 1) void sq_decode_kernel(SqDecodeArgs a) {
    constexpr int T = D / 16, S = D / 32;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kDecThreads / 64;
    const int v = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int RW = a.t.rec_words, RWS = 16 * RW + 4;    // +4: a window may run past the last record
    uint32_t* cb = reinterpret_cast<uint32_t*>(smem);                            // [width][256] (hi, lo)
    u32x4* At = reinterpret_cast<u32x4*>(smem + kCbRows * 256 * 4);              // [part][t][s][lane]
    uint32_t* stage = reinterpret_cast<uint32_t*>(smem + kCbRows * 256 * 4 + (size_t)2 * T * S * 1024) +
                      wave * NG * RWS;
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.dec_a) + (size_t)head * 2 * T * S * 64;
        for (int i = threadIdx.x; i < 2 * T * S * 64; i += kDecThreads) At[i] = src[i];
        const uint32_t* c = reinterpret_cast<const uint32_t*>(a.t.cb_hl);
        for (int i = threadIdx.x; i < kCbRows * 256; i += kDecThreads) cb[i] = c[i];
        for (int i = lane; i < NG * RWS; i += 64) stage[i] = 0u;
    }
    uint4 fd[S];
#pragma unroll
    for (int s = 0; s < S; ++s) fd[s] = a.t.fields[((size_t)head * S + s) * 4 + g];
    const float scale = a.t.dec_scale[head];
    __syncthreads();

    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint32_t* is = a.in + (size_t)st * a.n_tokens * RW;

    // records of the next NG tiles are fetched into registers one iteration ahead
    constexpr int NP = (16 * (D / 4 + 3) + 63) / 64;    // words per tile: 16 records of at most D/4 + 3 words
    uint32_t pre[NG][NP];
    auto fetch = [&](int64_t tile0) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t tq_ = tile0 + q;
            const int valid = tq_ < t_end ? (int)min((int64_t)16, a.n_tokens - tq_ * 16) : 0;
            fetch_words<NP>(is + (size_t)tq_ * 16 * RW, 16 * RW, valid * RW, lane, pre[q]);
        }
    };
    fetch(t_begin + (int64_t)wave * NG);
    for (int64_t tile = t_begin + (int64_t)wave * NG; tile < t_end; tile += (int64_t)nwaves * NG) {
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int j = 0; j < NP; ++j)
                if (lane + 64 * j < 16 * RW) stage[q * RWS + lane + 64 * j] = pre[q][j];
        fetch(tile + (int64_t)nwaves * NG);
        // k-step outer: the step's fields become the B operands of both tiles, and every A tile read
        // from LDS feeds NG x 3 independent products
        floatx4 acc[NG][T];
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[q][t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < S; ++s) {
            half8 Bh[NG], Bl[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                uint32_t ix[8];
                fields8(stage + q * RWS + v * RW, fd[s], ix);
                u32x4 hv, lv;
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const uint32_t p0 = cb[ix[i]], p1 = cb[ix[i + 1]];
                    hv[i / 2] = (p0 & 0xffffu) | (p1 << 16);
                    lv[i / 2] = (p0 >> 16) | (p1 & 0xffff0000u);
                }
                Bh[q] = as_half8(hv);
                Bl[q] = as_half8(lv);
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const half8 ah = as_half8(At[(t * S + s) * 64 + lane]);
                const half8 al = as_half8(At[((T + t) * S + s) * 64 + lane]);
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bh[q], acc[q][t], 0, 0, 0);
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bl[q], acc[q][t], 0, 0, 0);
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, Bh[q], acc[q][t], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t tok = (tile + q) * 16 + v;
            if (tile + q >= t_end || tok >= a.n_tokens) continue;
            const size_t o = ((size_t)st * a.n_tokens + tok) * D + 4 * g;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if constexpr (BF) {
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o + 16 * t) =
                        u32x2{bf16_pair(acc[q][t][0] * scale, acc[q][t][1] * scale),
                              bf16_pair(acc[q][t][2] * scale, acc[q][t][3] * scale)};
                } else {
                    *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + o + 16 * t) =
                        floatx4{acc[q][t][0] * scale, acc[q][t][1] * scale, acc[q][t][2] * scale, acc[q][t][3] * scale};
                }
            }
        }
    }
}

template <int D, bool BF>
static hipError_t launch_dec(const SqDecodeArgs& a, int num_cus, hipStream_t s) {
    constexpr int NG = 2;
    SqDecodeArgs b = a;
    const size_t lds = (size_t)kCbRows * 256 * 4 + (size_t)2 * (D / 16) * (D / 32) * 1024 +
                       (size_t)(kDecThreads / 64) * NG * (16 * a.t.rec_words + 4) * 4;
    if (lds > kLdsMax) return hipErrorInvalidValue;
    const void* kern = reinterpret_cast<const void*>(&sq_decode_kernel<D, BF, NG>);
    if (lds > 65536) {
        const hipError_t e = raise_lds(kern);
        if (e != hipSuccess) return e;
    }
    split_grid(b, kern, kDecThreads, lds, num_cus);
    hipLaunchKernelGGL((sq_decode_kernel<D, BF, NG>), dim3((unsigned)(b.n_streams * b.blocks_per_stream)),
                       dim3(kDecThreads), lds, s, b);
    return hipGetLastError();
}

hipError_t launch_sq_decode(const SqDecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s) {
    if (a.t.d == 64) return out_bf16 ? launch_dec<64, true>(a, num_cus, s) : launch_dec<64, false>(a, num_cus, s);
    return out_bf16 ? launch_dec<128, true>(a, num_cus, s) : launch_dec<128, false>(a, num_cus, s);
}

// ---------------------------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------------------------
// one block of D threads per (stream, padded query row): q'_k = σ_k Σ_j U[j][k] q_j in fp32, then
// scaled by 2^e (largest |q'| in [2^13, 2^14)) into an fp16 hi part and the fp16 remainder (together
// within ~2^-22 of the fp32 value); rows past n_q are zero
template <int D>
__global__ __launch_bounds__(D) void sq_qprep_kernel(SqScoresArgs a) {
    __shared__ float qs[D];
    __shared__ float red[D / 64];
    const int k = threadIdx.x;
    const int64_t row = blockIdx.x, st = row / a.nq_pad, i = row % a.nq_pad;
    const int head = (int)(st % a.t.n_heads);
    float qv = 0.0f;
    if (i < a.n_q) {
        const size_t o = ((size_t)st * a.n_q + i) * D + k;
        qv = a.q_bf16 ? u2f((uint32_t)static_cast<const uint16_t*>(a.q)[o] << 16) : static_cast<const float*>(a.q)[o];
    }
    qs[k] = qv;
    __syncthreads();
    const float* U = a.t.U32 + (size_t)head * D * D;
    float raw = 0.0f;
    for (int j = 0; j < D; ++j) raw = fmaf(U[(size_t)j * D + k], qs[j], raw);
    const float acc = raw * a.t.sigma[(size_t)head * D + k] * a.qmul;
    float m = fabsf(acc);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((k & 63) == 0) red[k >> 6] = m;
    __syncthreads();
    m = red[0];
    for (int w = 1; w < D / 64; ++w) m = fmaxf(m, red[w]);
    const int e = m > 0.0f ? 13 - ((int)((f2u(m) >> 23) & 0xffu) - 127) : 0;
    const float qv2 = __builtin_amdgcn_ldexpf(acc, e);
    const _Float16 qh = (_Float16)qv2;
    a.qp[(size_t)row * D + k] = qh;
    if (a.qplo) a.qplo[(size_t)row * D + k] = (_Float16)(qv2 - (float)qh);
    if (k == 0) a.qscale[row] = __builtin_amdgcn_ldexpf(1.0f, -e);
    if (a.t.m > 0) {
        // the selective sketch's side: p = S q_Z over the first 32 dimensions (zero rows and columns
        // beyond m and d_eff), in the first wave, fp16 with its own row scale
        __shared__ float qz[32];
        if (k < 32) qz[k] = raw * a.qmul;
        __syncthreads();
        if (k < 64) {
            const float* Srow = a.t.sk32 + ((size_t)head * 64 + k) * 32;
            float pv = 0.0f;
            for (int j = 0; j < 32; ++j) pv = fmaf(Srow[j], qz[j], pv);
            float mp = fabsf(pv);
            for (int o = 32; o > 0; o >>= 1) mp = fmaxf(mp, __shfl_xor(mp, o));
            const int e2 = mp > 0.0f ? 13 - ((int)((f2u(mp) >> 23) & 0xffu) - 127) : 0;
            const float pv2 = __builtin_amdgcn_ldexpf(pv, e2);
            const _Float16 ph = (_Float16)pv2;
            a.pp[(size_t)row * 64 + k] = ph;
            if (a.pplo) a.pplo[(size_t)row * 64 + k] = (_Float16)(pv2 - (float)ph);
            if (k == 0) a.pscale[row] = __builtin_amdgcn_ldexpf(1.2533141373155003f / (float)a.t.m, -e2);
        }
    }
}

constexpr int kScThreads = 256;

// Scores of 16 tokens (one wave tile) against all queries of the stream: A = the projected queries
// as fp16 hi + lo parts, B = the tokens' codebook values as hi + lo parts of c·2^12 (three products
// hi·hi + lo·hi + hi·lo); with the selective sketch, A = S q_Z as hi + lo parts and B = the exact ±1
// signs (two products).  Only the fp32 accumulation rounds, so the scores are fp32-accurate, also
// for one token or a cancelling score.
template <int D>
__global__ __launch_bounds__(kScThreads) void sq_scores_kernel(SqScoresArgs a) {
    constexpr int S = D / 32, QROW = D + 8;   // padded fp16 rows: 16 B apart in the banks
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kScThreads / 64;
    const int v = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int RW = a.t.rec_words, RWS = 16 * RW + 4;
    const int nqt = (int)(a.nq_pad / 16);
    const bool sk = a.t.m > 0;
    uint32_t* cb = reinterpret_cast<uint32_t*>(smem);                            // [width][256] fp16 (hi, lo)
    _Float16* qp = reinterpret_cast<_Float16*>(smem + kCbRows * 256 * 4);
    _Float16* qpl = qp + (size_t)a.nq_pad * QROW;
    float* qsc = reinterpret_cast<float*>(qpl + (size_t)a.nq_pad * QROW);
    // with the sketch: S q_Z rows (64 + 8 halves each, hi then lo), their scales and the byte -> ±1 table
    _Float16* ppl = reinterpret_cast<_Float16*>(qsc + a.nq_pad);
    _Float16* ppll = ppl + (sk ? a.nq_pad * 72 : 0);
    float* psc = reinterpret_cast<float*>(ppll + (sk ? a.nq_pad * 72 : 0));
    u32x4* pm = reinterpret_cast<u32x4*>(psc + (sk ? a.nq_pad : 0));
    uint32_t* stage = reinterpret_cast<uint32_t*>(pm + (sk ? 256 : 0)) + wave * RWS;
    {
        const _Float16* src = a.qp + (size_t)st * a.nq_pad * D;
        const _Float16* srl = a.qplo + (size_t)st * a.nq_pad * D;
        for (int i = threadIdx.x; i < a.nq_pad * D; i += kScThreads) {
            qp[(i / D) * QROW + i % D] = src[i];
            qpl[(i / D) * QROW + i % D] = srl[i];
        }
        for (int i = threadIdx.x; i < a.nq_pad; i += kScThreads) qsc[i] = a.qscale[(size_t)st * a.nq_pad + i];
        const uint32_t* c = reinterpret_cast<const uint32_t*>(a.t.cb_hl);
        for (int i = threadIdx.x; i < kCbRows * 256; i += kScThreads) cb[i] = c[i];
        if (sk) {
            const _Float16* ps = a.pp + (size_t)st * a.nq_pad * 64;
            const _Float16* psl = a.pplo + (size_t)st * a.nq_pad * 64;
            for (int i = threadIdx.x; i < a.nq_pad * 64; i += kScThreads) {
                ppl[(i / 64) * 72 + i % 64] = ps[i];
                ppll[(i / 64) * 72 + i % 64] = psl[i];
            }
            for (int i = threadIdx.x; i < a.nq_pad; i += kScThreads) psc[i] = a.pscale[(size_t)st * a.nq_pad + i];
            const u32x4* t = reinterpret_cast<const u32x4*>(a.t.pm1);
            for (int i = threadIdx.x; i < 256; i += kScThreads) pm[i] = t[i];
        }
        for (int i = lane; i < RWS; i += 64) stage[i] = 0u;
    }
    const uint32_t skoff = sk ? (uint32_t)a.t.sk_off[head] : 0u;
    uint4 fd[S];
#pragma unroll
    for (int s = 0; s < S; ++s) fd[s] = a.t.fields[((size_t)head * S + s) * 4 + g];
    __syncthreads();

    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint32_t* is = a.in + (size_t)st * a.n_tokens * RW;
    float* out = a.scores + (size_t)st * a.n_q * a.n_tokens;
    constexpr int NP = (16 * (D / 4 + 3) + 63) / 64;   // records of at most D/4 + 3 words
    uint32_t pre[NP];
    auto fetch = [&](int64_t tile) {
        const int valid = tile < t_end ? (int)min((int64_t)16, a.n_tokens - tile * 16) : 0;
        fetch_words<NP>(is + (size_t)tile * 16 * RW, 16 * RW, valid * RW, lane, pre);
    };
    fetch(t_begin + wave);
    for (int64_t tile = t_begin + wave; tile < t_end; tile += nwaves) {
#pragma unroll
        for (int j = 0; j < NP; ++j)
            if (lane + 64 * j < 16 * RW) stage[lane + 64 * j] = pre[j];
        fetch(tile + nwaves);
        half8 Bh[S], Bl[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            uint32_t ix[8];
            fields8(stage + v * RW, fd[s], ix);
            u32x4 hv, lv;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t e0 = cb[ix[i]], e1 = cb[ix[i + 1]];
                hv[i / 2] = (e0 & 0xffffu) | (e1 << 16);
                lv[i / 2] = (e0 >> 16) | (e1 & 0xffff0000u);
            }
            Bh[s] = as_half8(hv);
            Bl[s] = as_half8(lv);
        }
        // the sketch's ±1 operand (bits 32 s + 8 g + i of token v) and the token's fp16 norm
        half8 Bs[2];
        float rt = 0.0f;
        if (sk) {
            const uint32_t* rec = stage + v * RW;
#pragma unroll
            for (int s = 0; s < 2; ++s) Bs[s] = as_half8(pm[get_bits_at(rec, skoff + 32 * s + 8 * g, 8)]);
            rt = (float)__builtin_bit_cast(_Float16, (uint16_t)get_bits_at(rec, skoff + a.t.m, 16));
        }
        const int64_t tok = tile * 16 + v;
        for (int qt = 0; qt < nqt; ++qt) {
            floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f}, acs = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int o = (qt * 16 + v) * QROW + 32 * s + 8 * g;
                const half8 ah = *reinterpret_cast<const half8*>(qp + o);
                const half8 al = *reinterpret_cast<const half8*>(qpl + o);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bh[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, Bh[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bl[s], acc, 0, 0, 0);
            }
            if (sk) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int o = (qt * 16 + v) * 72 + 32 * s + 8 * g;
                    acs = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8*>(ppl + o), Bs[s], acs, 0, 0, 0);
                    acs = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8*>(ppll + o), Bs[s], acs, 0, 0, 0);
                }
            }
            if (tok < a.n_tokens) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = qt * 16 + 4 * g + r;
                    if (qi < a.n_q)
                        out[(size_t)qi * a.n_tokens + tok] = acc[r] * (qsc[qi] * (1.0f / 4096.0f)) + (sk ? acs[r] * psc[qi] * rt : 0.0f);
                }
            }
        }
    }
}

hipError_t launch_sq_qprep(const SqScoresArgs& a, hipStream_t s) {
    const unsigned rows = (unsigned)(a.n_streams * a.nq_pad);
    if (a.t.d == 64) hipLaunchKernelGGL((sq_qprep_kernel<64>), dim3(rows), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((sq_qprep_kernel<128>), dim3(rows), dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sq_scores(const SqScoresArgs& a, int num_cus, hipStream_t s) {
    SqScoresArgs b = a;
    hipError_t e = launch_sq_qprep(a, s);
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)kCbRows * 256 * 4 + (size_t)a.nq_pad * (a.t.d + 8) * 4 + (size_t)a.nq_pad * 4 +
                       (a.t.m > 0 ? (size_t)a.nq_pad * 72 * 4 + (size_t)a.nq_pad * 4 + 4096 : 0) +
                       (size_t)(kScThreads / 64) * (16 * a.t.rec_words + 4) * 4;
    if (lds > kLdsMax) return hipErrorInvalidValue;
    const void* kern = a.t.d == 64 ? reinterpret_cast<const void*>(&sq_scores_kernel<64>)
                                   : reinterpret_cast<const void*>(&sq_scores_kernel<128>);
    if (lds > 65536) {
        e = raise_lds(kern);
        if (e != hipSuccess) return e;
    }
    split_grid(b, kern, kScThreads, lds, num_cus);
    const dim3 grid((unsigned)(b.n_streams * b.blocks_per_stream));
    if (a.t.d == 64) hipLaunchKernelGGL((sq_scores_kernel<64>), grid, dim3(kScThreads), lds, s, b);
    else hipLaunchKernelGGL((sq_scores_kernel<128>), grid, dim3(kScThreads), lds, s, b);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// decode-attention
// ---------------------------------------------------------------------------------------------
// One wave per (stream, split) over 32-token chunks:
//   scores  D[token][query] = Σ_k c_K[token][k] · q'[query][k]  (A = the keys' codebook values from
//           their records, B = the projected queries, held in registers), already in base-2 units;
//   softmax online per query (running max and sum, the partial output rescaled when the max rises);
//   values  D[k][query] += Σ_t c_V[t][k] · p[t][query]: B = the weights exactly as the score product
//           left them (lane (query, g) holds tokens 4g + r of both 16-token halves, which is the
//           token order τ(g, i) used along the contraction), A = for dimension 16t + l%16 the value
//           fields of those 8 tokens, each read at the dimension's fixed bit offset.
// The partial outputs stay in the V basis without σ_V; the combine kernel merges the splits, then
// applies σ_V and U_V once per output row.
constexpr int kAttnThreads = 256;

template <int D, int RWM, bool SK>
__global__ __launch_bounds__(kAttnThreads, 2) void sq_attn_kernel(SqAttnArgs a) {
    constexpr int T = D / 16, S = D / 32;
    constexpr int NP = (32 * RWM + 63) / 64;           // record words of a 32-token chunk per lane
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    uint16_t* cb = reinterpret_cast<uint16_t*>(smem);                              // [width][256] fp16
    u32x4* pm = reinterpret_cast<u32x4*>(smem + kCbRows * 256 * 2);                // byte -> 8 x ±1 fp16
    const int RWk = a.tk.rec_words, RWv = a.tv.rec_words;
    const int WS = 32 * (RWk + RWv) + 4;
    uint32_t* sk = reinterpret_cast<uint32_t*>(smem + kCbRows * 256 * 2 + 4096) + wave * WS;
    uint32_t* sv = sk + 32 * RWk + 2;
    const int MK = SK ? a.tk.m : 0;   // the keys' sketch length
    {
        const uint16_t* c = reinterpret_cast<const uint16_t*>(a.tk.cb_h);
        for (int i = threadIdx.x; i < kCbRows * 256; i += kAttnThreads) cb[i] = c[i];
        if (MK > 0) {
            const u32x4* t = reinterpret_cast<const u32x4*>(a.tk.pm1);
            for (int i = threadIdx.x; i < 256; i += kAttnThreads) pm[i] = t[i];
        }
        for (int i = lane; i < WS; i += 64) sk[i] = 0u;
    }
    __syncthreads();
    const int64_t item = (int64_t)blockIdx.x * (kAttnThreads / 64) + wave;
    if (item >= a.n_streams * a.n_split) return;
    const int64_t st = item / a.n_split, sp = item % a.n_split;
    const int hk = (int)(st % a.hkv);
    int64_t len = a.n_tokens;
    if (a.lens) len = min(max((int64_t)a.lens[st / a.hkv], (int64_t)0), a.n_tokens);
    const int64_t t0 = sp * a.tps, t1 = min(t0 + a.tps, len);

    half8 Bq[S], Bql[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        Bq[s] = *reinterpret_cast<const half8*>(a.qp + ((size_t)st * 16 + n) * D + 32 * s + 8 * g);
        Bql[s] = *reinterpret_cast<const half8*>(a.qplo + ((size_t)st * 16 + n) * D + 32 * s + 8 * g);
    }
    const float qs = a.qscale[st * 16 + n];
    // the key sketch's query side (S q_Z of query n) and its scale
    half8 Bp[2];
    float pks = 0.0f;
    uint32_t skoff = 0u;
    if (MK > 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Bp[s] = *reinterpret_cast<const half8*>(a.pp + ((size_t)st * 16 + n) * 64 + 32 * s + 8 * g);
        pks = a.pscale[st * 16 + n];
        skoff = (uint32_t)a.tk.sk_off[hk];
    }
    uint4 fk[S];
#pragma unroll
    for (int s = 0; s < S; ++s) fk[s] = a.tk.fields[((size_t)hk * S + s) * 4 + g];
    uint32_t vm[T];   // value dimension 16t + n: bit offset << 16 | width << 26 (from its descriptor)
#pragma unroll
    for (int t = 0; t < T; ++t) vm[t] = f2u(a.tv.enc_desc[(size_t)hk * D + 16 * t + n].z);

    const uint32_t* ks = a.kin + (size_t)st * a.n_tokens * RWk;
    const uint32_t* vs = a.vin + (size_t)st * a.n_tokens * RWv;
    uint32_t pk[NP], pv[NP];
    auto fetch = [&](int64_t c0) {
        const int valid = c0 < t1 ? (int)min((int64_t)32, a.n_tokens - c0) : 0;
        fetch_words<NP>(ks + (size_t)c0 * RWk, 32 * RWk, valid * RWk, lane, pk);
        fetch_words<NP>(vs + (size_t)c0 * RWv, 32 * RWv, valid * RWv, lane, pv);
    };
    float m = -INFINITY, l = 0.0f;
    floatx4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    fetch(t0);
    for (int64_t c0 = t0; c0 < t1; c0 += 32) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            if (lane + 64 * j < 32 * RWk) sk[lane + 64 * j] = pk[j];
            if (lane + 64 * j < 32 * RWv) sv[lane + 64 * j] = pv[j];
        }
        fetch(c0 + 32);
        // scores of the two 16-token halves (the field descriptors pass through an empty asm each
        // chunk so that their decoded positions and widths are not kept live across the loop)
#pragma unroll
        for (int s = 0; s < S; ++s) asm volatile("" : "+v"(fk[s].x), "+v"(fk[s].y), "+v"(fk[s].z), "+v"(fk[s].w));
        float sc[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            floatx4 d4 = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                uint32_t ix[8];
                fields8(sk + (16 * h + n) * RWk, fk[s], ix);
                u32x4 hv;
#pragma unroll
                for (int i = 0; i < 8; i += 2) hv[i / 2] = (uint32_t)cb[ix[i]] | ((uint32_t)cb[ix[i + 1]] << 16);
                d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(hv), Bq[s], d4, 0, 0, 0);
                d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(hv), Bql[s], d4, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            float add4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (MK > 0) {   // sqrt(pi/2)/m · ||e_z|| · <S q_Z, 2σ - 1>, tokens 16h + n as A
                floatx4 dc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const half8 as = as_half8(pm[get_bits_at(sk + (16 * h + n) * RWk, skoff + 32 * s + 8 * g, 8)]);
                    dc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as, Bp[s], dc, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t rb = get_bits_at(sk + (16 * h + 4 * g + r) * RWk, skoff + (uint32_t)MK, 16);
                    add4[r] = dc[r] * pks * (float)__builtin_bit_cast(_Float16, (uint16_t)rb);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sc[h][r] = (c0 + 16 * h + 4 * g + r < t1) ? d4[r] * qs + add4[r] : -INFINITY;
        }
        // online softmax for query n (its 32 scores live on lanes n, n+16, n+32, n+48)
        float cm = sc[0][0];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) cm = fmaxf(cm, sc[h][r]);
        float x0 = cm, x1 = cm;
        xswap16(x0, x1);
        cm = fmaxf(x0, x1);
        x0 = cm;
        x1 = cm;
        xswap32(x0, x1);
        cm = fmaxf(x0, x1);
        const float mn = fmaxf(m, cm);
        const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mn);   // raw v_exp_f32
        float p[2][4], ps = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[h][r] = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[h][r] - mn);
                ps += p[h][r];
            }
        l = l * alpha + sum4(ps);
        m = mn;
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] *= alpha;
        const half8 P = half8{(_Float16)p[0][0], (_Float16)p[0][1], (_Float16)p[0][2], (_Float16)p[0][3],
                              (_Float16)p[1][0], (_Float16)p[1][1], (_Float16)p[1][2], (_Float16)p[1][3]};
        // values: dimension 16t + n of the tokens τ(g, i) = 4g + i (i < 4), 16 + 4g + i - 4 (i >= 4).
        // The word index goes through an empty asm each chunk so that its 8·T per-token forms are
        // not kept live across the loop.
        int zo = 0;
        asm volatile("" : "+v"(zo));
#pragma unroll
        for (int t = 0; t < T; ++t) asm volatile("" : "+v"(vm[t]));
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t off = (vm[t] >> 16) & 0x3ffu, wid = vm[t] >> 26;
            const uint32_t wi = off >> 5, sh = off & 31u, hi = wid << 8;
            u32x4 av;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                uint32_t c2[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int ii = i + k, tok = ii < 4 ? 4 * g + ii : 16 + 4 * g + ii - 4;
                    const uint32_t* w = sv + (zo + tok * RWv + (int)wi);
                    c2[k] = cb[hi | __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[1], w[0], sh), 0, wid)];
                }
                av[i / 2] = c2[0] | (c2[1] << 16);
            }
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(av), P, acc[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep each dimension tile's reads next to its product
        }
    }
    float* pp = a.part + ((size_t)item * 16 + n) * D;
#pragma unroll
    for (int t = 0; t < T; ++t)
        *reinterpret_cast<floatx4*>(pp + 16 * t + 4 * g) = acc[t];
    if (g == 0) *reinterpret_cast<float2*>(a.ml + ((size_t)item * 16 + n) * 2) = float2{m, l};
}

// one block of D threads per output row (b, h): merge the splits, scale by σ_V, rotate by U_V
template <int D>
__global__ __launch_bounds__(D) void sq_attn_combine_kernel(SqAttnArgs a) {
    __shared__ float y[D];
    const int k = threadIdx.x;
    const int64_t row = blockIdx.x, b = row / a.hq, h = row % a.hq;
    const int64_t hk = h / a.g, qi = h % a.g, st = b * a.hkv + hk;
    float M = -INFINITY;
    for (int64_t sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, a.ml[((st * a.n_split + sp) * 16 + qi) * 2]);
    float L = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
        for (int64_t sp = 0; sp < a.n_split; ++sp) {
            const size_t r = (size_t)(st * a.n_split + sp) * 16 + qi;
            const float w = exp2f(a.ml[r * 2] - M);
            L += a.ml[r * 2 + 1] * w;
            acc += a.part[r * D + k] * w;
        }
        acc = acc / L * a.tv.sigma[(size_t)hk * D + k];
    }
    y[k] = acc;
    __syncthreads();
    const float* U = a.tv.U32 + ((size_t)hk * D + k) * D;
    float o = 0.0f;
    for (int j = 0; j < D; ++j) o = fmaf(U[j], y[j], o);
    const size_t oi = (size_t)row * D + k;
    if (a.out_bf16) static_cast<__bf16*>(a.out)[oi] = (__bf16)o;
    else static_cast<float*>(a.out)[oi] = o;
}

template <int D, int RWM, bool SK>
static hipError_t launch_attn(const SqAttnArgs& a, hipStream_t s) {
    const size_t lds = (size_t)kCbRows * 256 * 2 + 4096 +
                       (size_t)(kAttnThreads / 64) * (32 * (a.tk.rec_words + a.tv.rec_words) + 4) * 4;
    const unsigned blocks = (unsigned)((a.n_streams * a.n_split + kAttnThreads / 64 - 1) / (kAttnThreads / 64));
    hipLaunchKernelGGL((sq_attn_kernel<D, RWM, SK>), dim3(blocks), dim3(kAttnThreads), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned rows = (unsigned)(a.n_streams / a.hkv * a.hq);
    hipLaunchKernelGGL((sq_attn_combine_kernel<D>), dim3(rows), dim3(D), 0, s, a);
    return hipGetLastError();
}

// records of up to 16 words (at most 4 bits per dimension on average at d = 128) take the smaller
// register prefetch, the larger d/4 words of 8-bit fields; with a key sketch (at most 64 bits and a
// 16-bit norm more) a middle size covers up to 5 bits per dimension at d = 128 without spilling
hipError_t launch_sq_attention(const SqAttnArgs& a, hipStream_t s) {
    const int rw = max(a.tk.rec_words, a.tv.rec_words);
    if (a.tk.m > 0) {
        if (a.tk.d == 64) return rw <= 8 ? launch_attn<64, 8, true>(a, s) : launch_attn<64, 19, true>(a, s);
        if (rw <= 16) return launch_attn<128, 16, true>(a, s);
        return rw <= 24 ? launch_attn<128, 24, true>(a, s) : launch_attn<128, 35, true>(a, s);
    }
    if (a.tk.d == 64) return rw <= 8 ? launch_attn<64, 8, false>(a, s) : launch_attn<64, 16, false>(a, s);
    return rw <= 16 ? launch_attn<128, 16, false>(a, s) : launch_attn<128, 32, false>(a, s);
}

}  // namespace tq
