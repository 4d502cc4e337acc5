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
//           registers.  Each index is OR-ed into a per-wave LDS record (ds_or), and the wave's 16
//           records are then written out linearly.
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

// bf16 pair (one word) times 2^sc into an fp16 pair (exact for every value within 2^-24 of the
// vector's largest; smaller ones are truncated to the fp16 subnormal grid)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_scaled(uint32_t w, int sc) {
    const float f0 = __builtin_amdgcn_ldexpf(u2f(w << 16), sc);
    const float f1 = __builtin_amdgcn_ldexpf(u2f(w & 0xffff0000u), sc);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1));
}

// field i of a lane's 8-field window: words d0..d3 from the record, rel < 96, width 1..8
__device__ __forceinline__ uint32_t window_field(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                                 uint32_t rel, uint32_t wid) {
    const uint32_t di = rel >> 5;
    const uint32_t lo = di == 0 ? d0 : (di == 1 ? d1 : d2);
    const uint32_t hi = di == 0 ? d1 : (di == 1 ? d2 : d3);
    return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(hi, lo, rel & 31u), 0, wid);
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

template <int D, int NG>
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
    uint32_t* stage = reinterpret_cast<uint32_t*>(smem + (size_t)2 * T * S * 1024 +
                                                  (size_t)((a.t.lds_grid_words + 3) / 4) * 16) +
                      wave * 16 * RW;
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.enc_b) + (size_t)head * 2 * T * S * 64;
        for (int i = threadIdx.x; i < 2 * T * S * 64; i += kEncThreads) Bt[i] = src[i];
        uint32_t* gw = reinterpret_cast<uint32_t*>(grid);
        for (int i = threadIdx.x; i < a.t.lds_grid_words; i += kEncThreads) gw[i] = a.t.grids[i];
        for (int i = lane; i < 16 * RW; i += 64) stage[i] = 0u;
    }
    float mul[T], add[T], cmax[T];
    uint32_t meta[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float4 dsc = a.t.enc_desc[(size_t)head * D + 16 * t + n];
        mul[t] = dsc.x;
        add[t] = dsc.y;
        meta[t] = f2u(dsc.z);
        cmax[t] = dsc.w;
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
            uint32_t e2 = 0u;
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t v = raw[q][s][w] & 0x7f807f80u;
                    e2 = max(e2, max(v & 0xffffu, v >> 16));
                }
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
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int q = 0; q < NG; ++q) acc[q][t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const half8 bh = as_half8(Bt[(t * S + s) * 64 + lane]);
                const half8 bl = as_half8(Bt[((T + t) * S + s) * 64 + lane]);
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[q][s], bh, acc[q][t], 0, 0, 0);
                    acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[q][s], bl, acc[q][t], 0, 0, 0);
                }
            }
        }

#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t tq_ = tile + q;
            if (tq_ >= t_end) break;
            int scr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) scr[r] = __shfl(sc[q], 4 * g + r);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t off = (meta[t] >> 16) & 0x3ffu, wid = meta[t] >> 26, goff = meta[t] & 0xffffu;
                const uint32_t wi = off >> 5, sh = off & 31u;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float z = __builtin_amdgcn_ldexpf(acc[q][t][r], -scr[r]);
                    const float ug = fmaf(z, mul[t], add[t]);
                    const int cell = (int)fminf(fmaxf(ug, 0.0f), cmax[t]);
                    const uint2 e = grid[goff + cell];
                    const uint32_t idx = e.y + (ug >= u2f(e.x) ? 1u : 0u);
                    uint32_t* rec = stage + (4 * g + r) * RW;
                    atomicOr(rec + wi, idx << sh);
                    if (sh + wid > 32u) atomicOr(rec + wi + 1, idx >> (32u - sh));
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

template <int D>
static hipError_t launch_enc(const SqEncodeArgs& a, int num_cus, hipStream_t s) {
    constexpr int NG = 2;
    SqEncodeArgs b = a;
    const size_t lds = (size_t)2 * (D / 16) * (D / 32) * 1024 + (size_t)((a.t.lds_grid_words + 3) / 4) * 16 +
                       (size_t)(kEncThreads / 64) * 16 * a.t.rec_words * 4;
    if (lds > kLdsMax) return hipErrorInvalidValue;
    const void* kern = reinterpret_cast<const void*>(&sq_encode_kernel<D, NG>);
    if (lds > 65536) {
        const hipError_t e = raise_lds(kern);
        if (e != hipSuccess) return e;
    }
    split_grid(b, kern, kEncThreads, lds, num_cus);
    hipLaunchKernelGGL((sq_encode_kernel<D, NG>), dim3((unsigned)(b.n_streams * b.blocks_per_stream)),
                       dim3(kEncThreads), lds, s, b);
    return hipGetLastError();
}

hipError_t launch_sq_encode(const SqEncodeArgs& a, int num_cus, hipStream_t s) {
    return a.t.d == 64 ? launch_enc<64>(a, num_cus, s) : launch_enc<128>(a, num_cus, s);
}

// ---------------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------------
constexpr int kDecThreads = 512;

template <int D, bool BF, int NG>
__global__ __launch_bounds__(kDecThreads, 1) void sq_decode_kernel(SqDecodeArgs a) {
    constexpr int T = D / 16, S = D / 32;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kDecThreads / 64;
    const int v = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int RW = a.t.rec_words, RWS = 16 * RW + 4;    // +4: a window may run past the last record
    u32x4* At = reinterpret_cast<u32x4*>(smem);                                  // [part][t][s][lane]
    uint32_t* cb = reinterpret_cast<uint32_t*>(smem + (size_t)2 * T * S * 1024);  // 510 (hi, lo) pairs
    uint32_t* stage = cb + 512 + wave * NG * RWS;
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.dec_a) + (size_t)head * 2 * T * S * 64;
        for (int i = threadIdx.x; i < 2 * T * S * 64; i += kDecThreads) At[i] = src[i];
        const uint32_t* c = reinterpret_cast<const uint32_t*>(a.t.cb_hl);
        for (int i = threadIdx.x; i < 510; i += kDecThreads) cb[i] = c[i];
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

    for (int64_t tile = t_begin + (int64_t)wave * NG; tile < t_end; tile += (int64_t)nwaves * NG) {
        // the NG tiles' records into LDS
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t tq_ = tile + q;
            const int64_t valid = tq_ < t_end ? min((int64_t)16, a.n_tokens - tq_ * 16) : 0;
            const uint32_t* src = is + (size_t)tq_ * 16 * RW;
            for (int i = lane; i < 16 * RW; i += 64) stage[q * RWS + i] = i < valid * RW ? src[i] : 0u;
        }
        half8 Bh[NG][S], Bl[NG][S];
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t* w = stage + q * RWS + v * RW + fd[s].x;
                const uint32_t d0 = w[0], d1 = w[1], d2 = w[2], d3 = w[3];
                u32x4 hv, lv;
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    uint32_t pr[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int ii = i + k;
                        const uint32_t rel = ((ii < 4 ? fd[s].y : fd[s].z) >> (8 * (ii & 3))) & 0xffu;
                        const uint32_t wid = (fd[s].w >> (4 * ii)) & 0xfu;
                        const uint32_t f = window_field(d0, d1, d2, d3, rel, wid);
                        pr[k] = cb[(1u << wid) - 2u + f];
                    }
                    hv[i / 2] = (pr[0] & 0xffffu) | (pr[1] << 16);
                    lv[i / 2] = (pr[0] >> 16) | (pr[1] & 0xffff0000u);
                }
                Bh[q][s] = as_half8(hv);
                Bl[q][s] = as_half8(lv);
            }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            floatx4 acc[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) acc[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const half8 ah = as_half8(At[(t * S + s) * 64 + lane]);
                const half8 al = as_half8(At[((T + t) * S + s) * 64 + lane]);
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bh[q][s], acc[q], 0, 0, 0);
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bl[q][s], acc[q], 0, 0, 0);
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, Bh[q][s], acc[q], 0, 0, 0);
                }
            }
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const int64_t tok = (tile + q) * 16 + v;
                if (tile + q >= t_end || tok >= a.n_tokens) continue;
                const size_t o = ((size_t)st * a.n_tokens + tok) * D + 16 * t + 4 * g;
                if constexpr (BF) {
                    uint32_t w0 = (f2u(acc[q][0] * scale) + 0x7fffu + ((f2u(acc[q][0] * scale) >> 16) & 1u)) >> 16;
                    uint32_t w1 = (f2u(acc[q][1] * scale) + 0x7fffu + ((f2u(acc[q][1] * scale) >> 16) & 1u)) >> 16;
                    uint32_t w2 = (f2u(acc[q][2] * scale) + 0x7fffu + ((f2u(acc[q][2] * scale) >> 16) & 1u)) >> 16;
                    uint32_t w3 = (f2u(acc[q][3] * scale) + 0x7fffu + ((f2u(acc[q][3] * scale) >> 16) & 1u)) >> 16;
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = u32x2{w0 | (w1 << 16), w2 | (w3 << 16)};
                } else {
                    *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + o) =
                        floatx4{acc[q][0] * scale, acc[q][1] * scale, acc[q][2] * scale, acc[q][3] * scale};
                }
            }
        }
    }
}

template <int D, bool BF>
static hipError_t launch_dec(const SqDecodeArgs& a, int num_cus, hipStream_t s) {
    constexpr int NG = 2;
    SqDecodeArgs b = a;
    const size_t lds = (size_t)2 * (D / 16) * (D / 32) * 1024 + 512 * 4 +
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
// scaled by 2^e (largest |q'| in [2^13, 2^14)) into fp16; rows past n_q are zero
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
    float acc = 0.0f;
    for (int j = 0; j < D; ++j) acc = fmaf(U[(size_t)j * D + k], qs[j], acc);
    acc *= a.t.sigma[(size_t)head * D + k];
    float m = fabsf(acc);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((k & 63) == 0) red[k >> 6] = m;
    __syncthreads();
    m = red[0];
    for (int w = 1; w < D / 64; ++w) m = fmaxf(m, red[w]);
    const int e = m > 0.0f ? 13 - ((int)((f2u(m) >> 23) & 0xffu) - 127) : 0;
    a.qp[(size_t)row * D + k] = (_Float16)__builtin_amdgcn_ldexpf(acc, e);
    if (k == 0) a.qscale[row] = __builtin_amdgcn_ldexpf(1.0f, -e);
}

constexpr int kScThreads = 256;

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
    _Float16* qp = reinterpret_cast<_Float16*>(smem);
    float* qsc = reinterpret_cast<float*>(smem + (size_t)a.nq_pad * QROW * 2);
    uint16_t* cb = reinterpret_cast<uint16_t*>(qsc + a.nq_pad);
    uint32_t* stage = reinterpret_cast<uint32_t*>(cb + 512) + wave * RWS;
    {
        const _Float16* src = a.qp + (size_t)st * a.nq_pad * D;
        for (int i = threadIdx.x; i < a.nq_pad * D; i += kScThreads) qp[(i / D) * QROW + i % D] = src[i];
        for (int i = threadIdx.x; i < a.nq_pad; i += kScThreads) qsc[i] = a.qscale[(size_t)st * a.nq_pad + i];
        const uint16_t* c = reinterpret_cast<const uint16_t*>(a.t.cb_h);
        for (int i = threadIdx.x; i < 510; i += kScThreads) cb[i] = c[i];
        for (int i = lane; i < RWS; i += 64) stage[i] = 0u;
    }
    uint4 fd[S];
#pragma unroll
    for (int s = 0; s < S; ++s) fd[s] = a.t.fields[((size_t)head * S + s) * 4 + g];
    __syncthreads();

    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint32_t* is = a.in + (size_t)st * a.n_tokens * RW;
    float* out = a.scores + (size_t)st * a.n_q * a.n_tokens;
    for (int64_t tile = t_begin + wave; tile < t_end; tile += nwaves) {
        const int64_t valid = min((int64_t)16, a.n_tokens - tile * 16);
        const uint32_t* src = is + (size_t)tile * 16 * RW;
        for (int i = lane; i < 16 * RW; i += 64) stage[i] = i < valid * RW ? src[i] : 0u;
        half8 B[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const uint32_t* w = stage + v * RW + fd[s].x;
            const uint32_t d0 = w[0], d1 = w[1], d2 = w[2], d3 = w[3];
            u32x4 hv;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                uint32_t pr[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int ii = i + k;
                    const uint32_t rel = ((ii < 4 ? fd[s].y : fd[s].z) >> (8 * (ii & 3))) & 0xffu;
                    const uint32_t wid = (fd[s].w >> (4 * ii)) & 0xfu;
                    pr[k] = cb[(1u << wid) - 2u + window_field(d0, d1, d2, d3, rel, wid)];
                }
                hv[i / 2] = pr[0] | (pr[1] << 16);
            }
            B[s] = as_half8(hv);
        }
        const int64_t tok = tile * 16 + v;
        for (int qt = 0; qt < nqt; ++qt) {
            floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const half8 aq = *reinterpret_cast<const half8*>(qp + (qt * 16 + v) * QROW + 32 * s + 8 * g);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, B[s], acc, 0, 0, 0);
            }
            if (tok < a.n_tokens) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = qt * 16 + 4 * g + r;
                    if (qi < a.n_q) out[(size_t)qi * a.n_tokens + tok] = acc[r] * qsc[qi];
                }
            }
        }
    }
}

hipError_t launch_sq_scores(const SqScoresArgs& a, int num_cus, hipStream_t s) {
    SqScoresArgs b = a;
    const unsigned rows = (unsigned)(a.n_streams * a.nq_pad);
    if (a.t.d == 64) hipLaunchKernelGGL((sq_qprep_kernel<64>), dim3(rows), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((sq_qprep_kernel<128>), dim3(rows), dim3(128), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)a.nq_pad * (a.t.d + 8) * 2 + (size_t)a.nq_pad * 4 + 512 * 2 +
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

}  // namespace tq
