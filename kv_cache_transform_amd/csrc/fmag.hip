// Fourier-magnitude codec kernels for gfx950 ("Fourier Magnitude KV Cache Quantization", forum
// thread, "Method": K -> FFT -> b-bit min-max magnitude, phase kept or quantised -> inverse FFT).
//
// MFMA layout (v_mfma_f32_16x16x32_f16): lane l supplies A[l%16][8(l/16)+i] and B[8(l/16)+i][l%16]
// and receives D[4(l/16)+r][l%16].
//
//   encode  D[vector][c] = Σ_j x[vector][j] · F[j][c]: the real DFT as a d x d real matrix (columns in
//           the spectrum-coordinate order of fmag_kernels.hpp), x exact in fp16 after a per-vector
//           power of two, F·2^8 as an fp16 hi + lo pair from LDS.  Lane (n, g) then holds the real
//           and imaginary parts of bins 16t' + n of vectors 4g + r: magnitude (sqrt), phase
//           (atan2), the vector's min and max over its 16-lane row (DPP), the b-bit magnitude and
//           p-bit (or bf16) phase fields, OR-ed over the lanes of a quad (a pair for bf16 phases)
//           and into the vector's record in LDS by the group's first lane.
//   decode  D[j][token] = Σ_c G[j][c] · X̂[token][c]: G the weighted inverse real DFT·2^e as hi + lo
//           from LDS, X̂ = (lo + q Δ)·(cos φ or sin φ) as hi + lo of the spectrum scaled per token by
//           a power of two; three products per step.
//   scores  D[query][token] = Σ_c q'[query][c] · X̂[token][c], q' = (w_c/d)·(F^T q)_c (Parseval).
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "common.hpp"
#include "fmag_kernels.hpp"

namespace tq {

namespace {

constexpr size_t kLdsMax = 163840;
constexpr float kPi = 3.14159265358979323846f;

__device__ __forceinline__ half8 as_h8(const u32x4& w) { return __builtin_bit_cast(half8, w); }

// atan2 in fp32: atan(t) on t = min/max in [0, 1] by an odd degree-15 polynomial (a weighted
// least-squares minimax fit to atan, |error| < 4e-8 on [0, 1]), then the octant reconstruction
// with the signs taken from the sign bits as atan2 does (±0 and ±π included); |error| < 5e-7 rad
__device__ __forceinline__ float atan2_poly(float y, float x) {
    const float ax = fabsf(x), ay = fabsf(y);
    const float mx = fmaxf(ax, ay), mn = fminf(ax, ay);
    const float t = mx > 0.0f ? mn * __builtin_amdgcn_rcpf(mx) : 0.0f;
    const float s = t * t;
    float p = -0.00405309209600091f;
    p = fmaf(p, s, 0.021856697276234627f);
    p = fmaf(p, s, -0.05590154603123665f);
    p = fmaf(p, s, 0.09641234576702118f);
    p = fmaf(p, s, -0.13908158242702484f);
    p = fmaf(p, s, 0.19946442544460297f);
    p = fmaf(p, s, -0.3332984447479248f);
    p = fmaf(p, s, 0.9999993443489075f);
    float r = p * t;
    if (ay > ax) r = 1.57079632679489662f - r;
    if (f2u(x) >> 31) r = kPi - r;
    return copysignf(r, y);
}

__device__ __forceinline__ uint32_t bf16x2_scaled_f16(uint32_t w, int sc) {
    const float f0 = __builtin_amdgcn_ldexpf(u2f(w << 16), sc);
    const float f1 = __builtin_amdgcn_ldexpf(u2f(w & 0xffff0000u), sc);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1));
}

__device__ __forceinline__ uint32_t pair_bf16(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// DPP within 16-lane rows
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dppf<0xb1>(v));
    v = fmaxf(v, dppf<0x4e>(v));
    v = fmaxf(v, dppf<0x141>(v));   // row_half_mirror
    return fmaxf(v, dppf<0x140>(v)); // row_mirror
}
__device__ __forceinline__ float row_min(float v) {
    v = fminf(v, dppf<0xb1>(v));
    v = fminf(v, dppf<0x4e>(v));
    v = fminf(v, dppf<0x141>(v));
    return fminf(v, dppf<0x140>(v));
}
__device__ __forceinline__ uint32_t quad_or4(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, true);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, true);
    return v;
}
__device__ __forceinline__ uint32_t pair_or(uint32_t v) {
    return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, true);
}

// OR bits [pos, pos + 32) of a record (v shifted into place, two words)
__device__ __forceinline__ void or_bits(uint32_t* rec, uint32_t pos, uint32_t v) {
    const uint64_t v64 = (uint64_t)v << (pos & 31u);
    atomicOr(rec + (pos >> 5), (uint32_t)v64);
    atomicOr(rec + (pos >> 5) + 1, (uint32_t)(v64 >> 32));
}

// `width` bits at bit `pos` of a record in LDS
__device__ __forceinline__ uint32_t get_field(const uint32_t* rec, uint32_t pos, uint32_t width) {
    const uint32_t* w = rec + (pos >> 5);
    return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[1], w[0], pos & 31u), 0, width);
}

template <int NP>
__device__ __forceinline__ void fetch_rec(const uint32_t* src, int count, int n_valid, int lane, uint32_t (&w)[NP]) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int i = lane + 64 * j;
        w[j] = (i < count && i < n_valid) ? src[i] : 0u;
    }
}

int occupancy(const void* k, int threads, size_t lds) {
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

hipError_t allow_lds(const void* kern) {
    static std::mutex mu;
    static std::map<const void*, bool> done;
    std::lock_guard<std::mutex> lock(mu);
    if (done[kern]) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (e == hipSuccess) done[kern] = true;
    return e;
}

template <typename Args>
void grid_split(Args& b, const void* kern, int threads, size_t lds, int num_cus) {
    const int64_t target = (int64_t)num_cus * occupancy(kern, threads, lds);
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
constexpr int kFmThreads = 512;

template <int D, bool PQ>   // PQ: p-bit phase indices (else bf16 phases); 4 waves per SIMD (two blocks per CU)
__global__ __launch_bounds__(kFmThreads, 4) void fmag_encode_kernel(FmEncodeArgs a) {
    constexpr int T = D / 16, S = D / 32, TH = T / 2, NB = D / 2 + 1;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kFmThreads / 64;
    const int n = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int RW = a.t.rec_words, WS = 16 * RW + 1;
    const uint32_t b = (uint32_t)a.t.b, p = (uint32_t)a.t.p;
    const float Lm1 = (float)((1 << b) - 1);
    const float pscale = (float)(1 << (p & 15u)) / (2.0f * kPi);
    u32x4* Bt = reinterpret_cast<u32x4*>(smem);
    uint32_t* stage = reinterpret_cast<uint32_t*>(smem + (size_t)2 * T * S * 1024) + wave * WS;
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.enc_b);
        for (int i = threadIdx.x; i < 2 * T * S * 64; i += kFmThreads) Bt[i] = src[i];
        for (int i = lane; i < WS; i += 64) stage[i] = 0u;
    }
    __syncthreads();

    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint16_t* xs = a.x + (size_t)st * a.n_tokens * D;
    uint32_t* os = a.out + (size_t)st * a.n_tokens * RW;

    for (int64_t tile = t_begin + wave; tile < t_end; tile += nwaves) {
        u32x4 raw[S];
        const int64_t tok = tile * 16 + n;
        if (tok < a.n_tokens) {
#pragma unroll
            for (int s = 0; s < S; ++s) raw[s] = *reinterpret_cast<const u32x4*>(xs + (size_t)tok * D + 32 * s + 8 * g);
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s) raw[s] = u32x4{0u, 0u, 0u, 0u};
        }
        // per-vector power-of-two scale into fp16 (largest |x| in [2^14, 2^15))
        uint32_t e2 = 0u;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t v = raw[s][w] & 0x7fff7fffu;
                e2 = max(e2, max(v & 0xffffu, v >> 16));
            }
        e2 &= 0x7f80u;
        uint32_t ea = e2, eb = e2;
        xswap16u(ea, eb);
        e2 = max(ea, eb);
        ea = e2;
        eb = e2;
        xswap32u(ea, eb);
        const int E = (int)(max(ea, eb) >> 7);
        const int sc = E == 0 ? 0 : 141 - E;
        half8 A[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            u32x4 h;
#pragma unroll
            for (int w = 0; w < 4; ++w) h[w] = bf16x2_scaled_f16(raw[s][w], sc);
            A[s] = as_h8(h);
        }
        floatx4 acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[s], as_h8(Bt[(t * S + s) * 64 + lane]), acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[s], as_h8(Bt[((T + t) * S + s) * 64 + lane]), acc[t], 0, 0, 0);
            }
        // vector 4g + r: its scale sits in lane 4g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int scr = __shfl(sc, 4 * g + r);
            float mag[TH], ph[TH], nyq = 0.0f;
            float lo = INFINITY, hi = 0.0f;
#pragma unroll
            for (int t = 0; t < TH; ++t) {
                const float re = __builtin_amdgcn_ldexpf(acc[t][r], -(8 + scr));
                float im = __builtin_amdgcn_ldexpf(acc[t + TH][r], -(8 + scr));
                if (t == 0 && n == 0) {   // the Im X_0 slot carries Re X_{d/2}
                    nyq = im;
                    im = 0.0f;
                }
                mag[t] = __builtin_amdgcn_sqrtf(fmaf(re, re, im * im));
                ph[t] = atan2_poly(im, re);
                lo = fminf(lo, mag[t]);
                hi = fmaxf(hi, mag[t]);
            }
            if (n == 0) {
                lo = fminf(lo, fabsf(nyq));
                hi = fmaxf(hi, fabsf(nyq));
            }
            lo = row_min(lo);
            hi = row_max(hi);
            const float inv = hi > lo ? Lm1 / (hi - lo) : 0.0f;
            uint32_t* rec = stage + (4 * g + r) * RW;
#pragma unroll
            for (int t = 0; t < TH; ++t) {
                const uint32_t kb = (uint32_t)(16 * t + n);
                const uint32_t qv = (uint32_t)fminf(floorf((mag[t] - lo) * inv + 0.5f), Lm1);
                const uint32_t qg = quad_or4(qv << ((n & 3) * b));
                if ((n & 3) == 0) or_bits(rec, kb * b, qg);
                if constexpr (PQ) {
                    const uint32_t pv = (uint32_t)(int)floorf((ph[t] + kPi) * pscale + 0.5f) & ((1u << p) - 1u);
                    const uint32_t pg = quad_or4(pv << ((n & 3) * p));
                    if ((n & 3) == 0) or_bits(rec, NB * b + kb * p, pg);
                } else {
                    const uint32_t pv = (f2u(ph[t]) + 0x7fffu + ((f2u(ph[t]) >> 16) & 1u)) >> 16;   // bf16, nearest even
                    const uint32_t pg = pair_or(pv << ((n & 1) * 16));
                    if ((n & 1) == 0) or_bits(rec, NB * b + kb * 16, pg);
                }
            }
            if (n == 0) {   // the Nyquist bin (real: phase 0 or π) and the min-max range
                const float m = fabsf(nyq);
                const uint32_t qv = (uint32_t)fminf(floorf((m - lo) * inv + 0.5f), Lm1);
                const float phn = atan2_poly(0.0f, nyq);
                uint32_t pv;
                if constexpr (PQ) pv = (uint32_t)(int)floorf((phn + kPi) * pscale + 0.5f) & ((1u << p) - 1u);
                else pv = (f2u(phn) + 0x7fffu + ((f2u(phn) >> 16) & 1u)) >> 16;
                or_bits(rec, (uint32_t)(D / 2) * b, qv);
                or_bits(rec, NB * b + (uint32_t)(D / 2) * p, pv);
                rec[RW - 2] = f2u(lo);
                rec[RW - 1] = f2u(hi);
            }
        }
        const int64_t valid = min((int64_t)16, a.n_tokens - tile * 16);
        uint32_t* dst = os + (size_t)tile * 16 * RW;
        for (int i = lane; i < 16 * RW; i += 64) {
            const uint32_t v = stage[i];
            stage[i] = 0u;
            if (i < valid * RW) dst[i] = v;
        }
    }
}

template <int D, bool PQ>
static hipError_t launch_fenc(const FmEncodeArgs& a, int num_cus, hipStream_t s) {
    FmEncodeArgs b = a;
    const size_t lds = (size_t)2 * (D / 16) * (D / 32) * 1024 + (size_t)(kFmThreads / 64) * (16 * a.t.rec_words + 1) * 4;
    const void* kern = reinterpret_cast<const void*>(&fmag_encode_kernel<D, PQ>);
    if (lds > 65536) {
        const hipError_t e = allow_lds(kern);
        if (e != hipSuccess) return e;
    }
    grid_split(b, kern, kFmThreads, lds, num_cus);
    hipLaunchKernelGGL((fmag_encode_kernel<D, PQ>), dim3((unsigned)(b.n_streams * b.blocks_per_stream)), dim3(kFmThreads),
                       lds, s, b);
    return hipGetLastError();
}

hipError_t launch_fmag_encode(const FmEncodeArgs& a, int num_cus, hipStream_t s) {
    const bool pq = a.t.p <= 8;
    if (a.t.d == 64) return pq ? launch_fenc<64, true>(a, num_cus, s) : launch_fenc<64, false>(a, num_cus, s);
    return pq ? launch_fenc<128, true>(a, num_cus, s) : launch_fenc<128, false>(a, num_cus, s);
}

// ---------------------------------------------------------------------------------------------
// spectrum coordinates of a record (decode and scores)
// ---------------------------------------------------------------------------------------------
// Lane (v, g) of k-step s supplies coordinates c = 32s + 8g + i (i = 0..7) of token v: for s < S/2
// the real parts of bins κ = c, else the imaginary parts of bins κ = c - d/2, whose first slot
// (g = 0, i = 0) is the real Nyquist bin.  Values are X̂ = (lo + q Δ)·(cos or sin of the phase),
// times 2^es (es from the token's hi, so |X̂|·2^es < 2^15).
template <int D, bool PQ>
__device__ __forceinline__ void spectrum8(const uint32_t* rec, int RW, uint32_t b, uint32_t p, int s, int g,
                                          const float* cs, float (&out)[8], int& es) {
    constexpr int S = D / 32, NB = D / 2 + 1;
    const float lo = u2f(rec[RW - 2]), hi = u2f(rec[RW - 1]);
    const float delta = (hi - lo) * (1.0f / (float)((1 << b) - 1));   // the reciprocal is loop-invariant
    es = hi > 0.0f ? 141 - (int)((f2u(hi) >> 23) & 0xffu) : 0;
    const bool im = s >= S / 2;
    const uint32_t k0 = (uint32_t)(32 * (im ? s - S / 2 : s) + 8 * g);
    // the 8 bins' fields are contiguous: one 64-bit window of magnitudes (8 b <= 64 bits) and one or
    // two of phases (8 p <= 128 bits), each from three record words
    auto window = [&](uint32_t pos) {
        const uint32_t* w = rec + (pos >> 5);
        const uint32_t sh = pos & 31u;
        return ((uint64_t)__builtin_amdgcn_alignbit(w[2], w[1], sh) << 32) | __builtin_amdgcn_alignbit(w[1], w[0], sh);
    };
    const uint64_t mw = window(k0 * b);
    const uint32_t ppos = (uint32_t)NB * b + k0 * p;
    const uint64_t pw0 = window(ppos);
    const uint64_t pw1 = PQ ? 0ull : window(ppos + 64u);
    const uint32_t mmask = (1u << b) - 1u;
    const uint64_t pmask = (1ull << p) - 1ull;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool nyq = s == S / 2 && g == 0 && i == 0;   // coordinate d/2 only: the real Nyquist bin
        uint32_t mf = (uint32_t)(mw >> (i * b)) & mmask;
        uint32_t pf;
        if constexpr (PQ) pf = (uint32_t)((pw0 >> (i * p)) & pmask);
        else pf = (uint32_t)((i < 4 ? pw0 >> (16 * i) : pw1 >> (16 * (i - 4))) & 0xffffu);
        if (nyq) {
            mf = get_field(rec, (uint32_t)(D / 2) * b, b);
            pf = get_field(rec, (uint32_t)NB * b + (uint32_t)(D / 2) * p, p);
        }
        const float mag = fmaf((float)mf, delta, lo);
        float trig;
        if constexpr (PQ) {
            trig = cs[2 * pf + ((im && !nyq) ? 1 : 0)];
        } else {
            const float ph = u2f(pf << 16);
            trig = (im && !nyq) ? __sinf(ph) : __cosf(ph);
        }
        out[i] = __builtin_amdgcn_ldexpf(mag * trig, es);
    }
}

// ---------------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------------
template <int D, bool BF, bool PQ>
__global__ __launch_bounds__(kFmThreads, 1) void fmag_decode_kernel(FmDecodeArgs a) {
    constexpr int T = D / 16, S = D / 32, NP = (16 * (D / 2) + 63) / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kFmThreads / 64;
    const int v = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int RW = a.t.rec_words, RWS = 16 * RW + 2;
    const uint32_t b = (uint32_t)a.t.b, p = (uint32_t)a.t.p;
    float* cs = reinterpret_cast<float*>(smem);                                     // 512 floats
    u32x4* At = reinterpret_cast<u32x4*>(smem + 2048);
    uint32_t* stage = reinterpret_cast<uint32_t*>(smem + 2048 + (size_t)2 * T * S * 1024) + wave * RWS;
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.dec_a);
        for (int i = threadIdx.x; i < 2 * T * S * 64; i += kFmThreads) At[i] = src[i];
        if (p <= 8u)
            for (int i = threadIdx.x; i < (2 << p); i += kFmThreads) cs[i] = a.t.cs[i];
        for (int i = lane; i < RWS; i += 64) stage[i] = 0u;
    }
    __syncthreads();
    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint32_t* is = a.in + (size_t)st * a.n_tokens * RW;
    uint32_t pre[NP];
    auto fetch = [&](int64_t tile) {
        const int valid = tile < t_end ? (int)min((int64_t)16, a.n_tokens - tile * 16) : 0;
        fetch_rec<NP>(is + (size_t)tile * 16 * RW, 16 * RW, valid * RW, lane, pre);
    };
    fetch(t_begin + wave);
    for (int64_t tile = t_begin + wave; tile < t_end; tile += nwaves) {
#pragma unroll
        for (int j = 0; j < NP; ++j)
            if (lane + 64 * j < 16 * RW) stage[lane + 64 * j] = pre[j];
        fetch(tile + nwaves);
        floatx4 acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        int es = 0;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            float x8[8];
            spectrum8<D, PQ>(stage + v * RW, RW, b, p, s, g, cs, x8, es);
            u32x4 hv, lv;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const _Float16 h0 = (_Float16)x8[i], h1 = (_Float16)x8[i + 1];
                const _Float16 l0 = (_Float16)(x8[i] - (float)h0), l1 = (_Float16)(x8[i + 1] - (float)h1);
                hv[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                lv[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const half8 ah = as_h8(At[(t * S + s) * 64 + lane]);
                const half8 al = as_h8(At[((T + t) * S + s) * 64 + lane]);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_h8(hv), acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_h8(lv), acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, as_h8(hv), acc[t], 0, 0, 0);
            }
        }
        const int64_t tok = tile * 16 + v;
        if (tok >= a.n_tokens) continue;
        const float scale = __builtin_amdgcn_ldexpf(a.t.dec_scale, -es);
        const size_t o = ((size_t)st * a.n_tokens + tok) * D + 4 * g;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if constexpr (BF) {
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o + 16 * t) =
                    u32x2{pair_bf16(acc[t][0] * scale, acc[t][1] * scale), pair_bf16(acc[t][2] * scale, acc[t][3] * scale)};
            } else {
                *reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + o + 16 * t) =
                    floatx4{acc[t][0] * scale, acc[t][1] * scale, acc[t][2] * scale, acc[t][3] * scale};
            }
        }
    }
}

template <int D, bool BF, bool PQ>
static hipError_t launch_fdec(const FmDecodeArgs& a, int num_cus, hipStream_t s) {
    FmDecodeArgs b = a;
    const size_t lds = 2048 + (size_t)2 * (D / 16) * (D / 32) * 1024 + (size_t)(kFmThreads / 64) * (16 * a.t.rec_words + 2) * 4;
    const void* kern = reinterpret_cast<const void*>(&fmag_decode_kernel<D, BF, PQ>);
    if (lds > 65536) {
        const hipError_t e = allow_lds(kern);
        if (e != hipSuccess) return e;
    }
    grid_split(b, kern, kFmThreads, lds, num_cus);
    hipLaunchKernelGGL((fmag_decode_kernel<D, BF, PQ>), dim3((unsigned)(b.n_streams * b.blocks_per_stream)), dim3(kFmThreads),
                       lds, s, b);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fdec_d(const FmDecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s) {
    if (a.t.p <= 8) return out_bf16 ? launch_fdec<D, true, true>(a, num_cus, s) : launch_fdec<D, false, true>(a, num_cus, s);
    return out_bf16 ? launch_fdec<D, true, false>(a, num_cus, s) : launch_fdec<D, false, false>(a, num_cus, s);
}

hipError_t launch_fmag_decode(const FmDecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s) {
    return a.t.d == 64 ? launch_fdec_d<64>(a, out_bf16, num_cus, s) : launch_fdec_d<128>(a, out_bf16, num_cus, s);
}

// ---------------------------------------------------------------------------------------------
// scores (the query side comes from the SpectralQuant query-prep kernel with U = the DFT matrix
// and σ_c = w_c/d)
// ---------------------------------------------------------------------------------------------
constexpr int kFsThreads = 256;

template <int D, bool PQ>
__global__ __launch_bounds__(kFsThreads) void fmag_scores_kernel(FmScoresArgs a) {
    constexpr int S = D / 32, QROW = D + 8, NP = (16 * (D / 2) + 63) / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = kFsThreads / 64;
    const int v = lane & 15, g = lane >> 4;
    const int64_t st = blockIdx.x / a.blocks_per_stream, blk = blockIdx.x % a.blocks_per_stream;
    const int RW = a.t.rec_words, RWS = 16 * RW + 2;
    const uint32_t b = (uint32_t)a.t.b, p = (uint32_t)a.t.p;
    const int nqt = (int)(a.nq_pad / 16);
    float* cs = reinterpret_cast<float*>(smem);
    _Float16* qp = reinterpret_cast<_Float16*>(smem + 2048);
    _Float16* qpl = qp + (size_t)a.nq_pad * QROW;
    float* qsc = reinterpret_cast<float*>(smem + 2048 + (size_t)a.nq_pad * QROW * 4);
    uint32_t* stage = reinterpret_cast<uint32_t*>(qsc + a.nq_pad) + wave * RWS;
    {
        const _Float16* src = a.qp + (size_t)st * a.nq_pad * D;
        const _Float16* srl = a.qplo + (size_t)st * a.nq_pad * D;
        for (int i = threadIdx.x; i < a.nq_pad * D; i += kFsThreads) {
            qp[(i / D) * QROW + i % D] = src[i];
            qpl[(i / D) * QROW + i % D] = srl[i];
        }
        for (int i = threadIdx.x; i < a.nq_pad; i += kFsThreads) qsc[i] = a.qscale[(size_t)st * a.nq_pad + i];
        if (p <= 8u)
            for (int i = threadIdx.x; i < (2 << p); i += kFsThreads) cs[i] = a.t.cs[i];
        for (int i = lane; i < RWS; i += 64) stage[i] = 0u;
    }
    __syncthreads();
    const int64_t t_begin = blk * a.tiles_per_block;
    const int64_t t_end = min(t_begin + a.tiles_per_block, a.tiles_per_stream);
    const uint32_t* is = a.in + (size_t)st * a.n_tokens * RW;
    float* out = a.scores + (size_t)st * a.n_q * a.n_tokens;
    uint32_t pre[NP];
    auto fetch = [&](int64_t tile) {
        const int valid = tile < t_end ? (int)min((int64_t)16, a.n_tokens - tile * 16) : 0;
        fetch_rec<NP>(is + (size_t)tile * 16 * RW, 16 * RW, valid * RW, lane, pre);
    };
    fetch(t_begin + wave);
    for (int64_t tile = t_begin + wave; tile < t_end; tile += nwaves) {
#pragma unroll
        for (int j = 0; j < NP; ++j)
            if (lane + 64 * j < 16 * RW) stage[lane + 64 * j] = pre[j];
        fetch(tile + nwaves);
        // the token's spectrum entries as fp16 hi + lo parts (three products with the query's parts:
        // fp32-accurate scores)
        half8 B[S], BL[S];
        int es = 0;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            float x8[8];
            spectrum8<D, PQ>(stage + v * RW, RW, b, p, s, g, cs, x8, es);
            u32x4 hv, lv;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const _Float16 h0 = (_Float16)x8[i], h1 = (_Float16)x8[i + 1];
                hv[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                lv[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(x8[i] - (float)h0)) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(x8[i + 1] - (float)h1)) << 16);
            }
            B[s] = as_h8(hv);
            BL[s] = as_h8(lv);
        }
        const int64_t tok = tile * 16 + v;
        const float tsc = __builtin_amdgcn_ldexpf(1.0f, -es);
        for (int qt = 0; qt < nqt; ++qt) {
            floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int o = (qt * 16 + v) * QROW + 32 * s + 8 * g;
                const half8 aq = *reinterpret_cast<const half8*>(qp + o);
                const half8 al = *reinterpret_cast<const half8*>(qpl + o);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, B[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, B[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, BL[s], acc, 0, 0, 0);
            }
            if (tok < a.n_tokens) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = qt * 16 + 4 * g + r;
                    if (qi < a.n_q) out[(size_t)qi * a.n_tokens + tok] = acc[r] * qsc[qi] * tsc;
                }
            }
        }
    }
}

template <int D, bool PQ>
static hipError_t launch_fsc(const FmScoresArgs& a, int num_cus, hipStream_t s) {
    FmScoresArgs b = a;
    const size_t lds = 2048 + (size_t)a.nq_pad * (D + 8) * 4 + (size_t)a.nq_pad * 4 +
                       (size_t)(kFsThreads / 64) * (16 * a.t.rec_words + 2) * 4;
    const void* kern = reinterpret_cast<const void*>(&fmag_scores_kernel<D, PQ>);
    if (lds > 65536) {
        const hipError_t e = allow_lds(kern);
        if (e != hipSuccess) return e;
    }
    grid_split(b, kern, kFsThreads, lds, num_cus);
    hipLaunchKernelGGL((fmag_scores_kernel<D, PQ>), dim3((unsigned)(b.n_streams * b.blocks_per_stream)),
                       dim3(kFsThreads), lds, s, b);
    return hipGetLastError();
}

hipError_t launch_fmag_scores(const FmScoresArgs& a, int num_cus, hipStream_t s) {
    const bool pq = a.t.p <= 8;
    if (a.t.d == 64) return pq ? launch_fsc<64, true>(a, num_cus, s) : launch_fsc<64, false>(a, num_cus, s);
    return pq ? launch_fsc<128, true>(a, num_cus, s) : launch_fsc<128, false>(a, num_cus, s);
}

// ---------------------------------------------------------------------------------------------
// decode-attention
// ---------------------------------------------------------------------------------------------
// One wave per (stream, split) over 32-token chunks, like the SpectralQuant attention, with the
// reconstructed spectra in place of codebook values (the inverse FFT is linear, so Σ_t p_t x̂_t is
// the inverse FFT of Σ_t p_t X̂_t):
//   scores  D[token][query] = Σ_c X̂_K[token][c]·q'[query][c]: A = the keys' spectrum coordinates
//           (per token times 2^es), B = the projected queries, both as fp16 hi + lo pairs (three
//           products: the scores carry about 2^-21 relative error, so the softmax of heavy-tailed
//           keys keeps its precision); each row then scaled by its token's 2^-es, in base-2 units;
//   softmax online per query;
//   values  D[c][query] += Σ_t X̂_V[t][c]·p[t][query]: B = the weights as the score product left
//           them (tokens τ(g, i) = 4g + i, 16 + 4g + i - 4 along the contraction), A = coordinate
//           16t + l%16 of those 8 tokens, all scaled by one power of two per chunk (from the chunk's
//           largest magnitude) that the fp32 accumulation undoes; the weights as fp16 hi + lo.
// The combine merges the splits and applies the weighted inverse real DFT once per output row.
constexpr int kFaThreads = 256;

template <bool PQ>
__device__ __forceinline__ float phase_trig(const uint32_t* rec, uint32_t pos, uint32_t p, bool sine, const float* cs) {
    const uint32_t pf = get_field(rec, pos, p);
    if constexpr (PQ) return cs[2 * pf + (sine ? 1 : 0)];
    const float ph = u2f(pf << 16);
    return sine ? __sinf(ph) : __cosf(ph);
}

template <int D, int RWM, bool PQK, bool PQV>
__global__ __launch_bounds__(kFaThreads, RWM <= 28 ? 3 : 2) void fmag_attn_kernel(FmAttnArgs a) {
    constexpr int T = D / 16, S = D / 32, NB = D / 2 + 1;
    constexpr int NP = (32 * RWM + 63) / 64;           // record words of a 32-token chunk per lane
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    float* csk = reinterpret_cast<float*>(smem);       // [256][2] cos, sin of the K phase levels
    float* csv = csk + 512;                            // the V phase levels
    const int RWk = a.tk.rec_words, RWv = a.tv.rec_words;
    const int WS = 32 * (RWk + RWv) + 4;
    _Float16* qlo = reinterpret_cast<_Float16*>(smem + 4096) + wave * (16 * D);   // this wave's q' remainders
    uint32_t* sk = reinterpret_cast<uint32_t*>(smem + 4096 + (kFaThreads / 64) * 16 * D * 2) + wave * WS;
    uint32_t* sv = sk + 32 * RWk + 2;
    const uint32_t bk = (uint32_t)a.tk.b, pk_ = (uint32_t)a.tk.p, bv = (uint32_t)a.tv.b, pv_ = (uint32_t)a.tv.p;
    {
        if (PQK)
            for (int i = threadIdx.x; i < (2 << pk_); i += kFaThreads) csk[i] = a.tk.cs[i];
        if (PQV)
            for (int i = threadIdx.x; i < (2 << pv_); i += kFaThreads) csv[i] = a.tv.cs[i];
        for (int i = lane; i < WS; i += 64) sk[i] = 0u;
    }
    __syncthreads();
    const int64_t item = (int64_t)blockIdx.x * (kFaThreads / 64) + wave;
    if (item >= a.n_streams * a.n_split) return;
    const int64_t st = item / a.n_split, sp = item % a.n_split;
    int64_t len = a.n_tokens;
    if (a.lens) len = min(max((int64_t)a.lens[st / a.hkv], (int64_t)0), a.n_tokens);
    const int64_t t0 = sp * a.tps, t1 = min(t0 + a.tps, len);

    half8 Bq[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        Bq[s] = *reinterpret_cast<const half8*>(a.qp + ((size_t)st * 16 + n) * D + 32 * s + 8 * g);
        *reinterpret_cast<half8*>(qlo + n * D + 32 * s + 8 * g) =
            *reinterpret_cast<const half8*>(a.qplo + ((size_t)st * 16 + n) * D + 32 * s + 8 * g);
    }
    const float qs = a.qscale[st * 16 + n];
    const float vden = 1.0f / (float)((1 << bv) - 1);

    const uint32_t* ks = a.kin + (size_t)st * a.n_tokens * RWk;
    const uint32_t* vs = a.vin + (size_t)st * a.n_tokens * RWv;
    uint32_t pk[NP], pv[NP];
    auto fetch = [&](int64_t c0) {
        const int valid = c0 < t1 ? (int)min((int64_t)32, a.n_tokens - c0) : 0;
        fetch_rec<NP>(ks + (size_t)c0 * RWk, 32 * RWk, valid * RWk, lane, pk);
        fetch_rec<NP>(vs + (size_t)c0 * RWv, 32 * RWv, valid * RWv, lane, pv);
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
        // the lane indices pass through an empty asm each chunk so that the field positions derived
        // from them are recomputed here instead of being kept live across the loop
        int gl = g, nl = n;
        asm volatile("" : "+v"(gl), "+v"(nl));
        // scores of the two 16-token halves
        float sc[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            floatx4 d4 = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                float x8[8];
                int es;
                spectrum8<D, PQK>(sk + (16 * h + nl) * RWk, RWk, bk, pk_, s, gl, csk, x8, es);
                u32x4 hv, lv;
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const _Float16 h0 = (_Float16)x8[i], h1 = (_Float16)x8[i + 1];
                    hv[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                    lv[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(x8[i] - (float)h0)) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(x8[i + 1] - (float)h1)) << 16);
                }
                const half8 bl = *reinterpret_cast<const half8*>(qlo + nl * D + 32 * s + 8 * gl);
                d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(hv), Bq[s], d4, 0, 0, 0);
                d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(lv), Bq[s], d4, 0, 0, 0);
                d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(hv), bl, d4, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);   // one k-step's spectrum at a time
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 16 * h + 4 * gl + r;
                const float hi = u2f(sk[tok * RWk + RWk - 1]);
                const int es = hi > 0.0f ? 141 - (int)((f2u(hi) >> 23) & 0xffu) : 0;
                sc[h][r] = (c0 + tok < t1) ? d4[r] * qs * __builtin_amdgcn_ldexpf(1.0f, -es) : -INFINITY;
            }
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
        float p[2][4], psum = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[h][r] = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[h][r] - mn);
                psum += p[h][r];
            }
        l = l * alpha + sum4(psum);
        m = mn;
        half8 P, PL;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float pf = p[i >> 2][i & 3];
            P[i] = (_Float16)pf;
            PL[i] = (_Float16)(pf - (float)P[i]);
        }
        // values: one power of two for the chunk from its largest magnitude (every |X̂| <= hi)
        float hm = row_max(u2f(sv[(lane & 31) * RWv + RWv - 1]));   // 16 tokens per row, then both rows
        x0 = hm;
        x1 = hm;
        xswap16(x0, x1);
        hm = fmaxf(x0, x1);
        const int ev = hm > 0.0f ? 141 - (int)((f2u(hm) >> 23) & 0xffu) : 0;
        const float vsc = __builtin_amdgcn_ldexpf(1.0f, -ev);
        float vlo[8], vdl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = i < 4 ? 4 * gl + i : 16 + 4 * gl + i - 4;
            vlo[i] = u2f(sv[tok * RWv + RWv - 2]);
            vdl[i] = (u2f(sv[tok * RWv + RWv - 1]) - vlo[i]) * vden;
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int c = 16 * t + nl;
            const bool im = c > D / 2;
            const uint32_t kb = (uint32_t)(c <= D / 2 ? c : c - D / 2);
            u32x4 av;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                uint32_t h2[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int ii = i + k, tok = ii < 4 ? 4 * gl + ii : 16 + 4 * gl + ii - 4;
                    const uint32_t* rec = sv + tok * RWv;
                    const float mag = fmaf((float)get_field(rec, kb * bv, bv), vdl[ii], vlo[ii]);
                    const float trig = phase_trig<PQV>(rec, (uint32_t)NB * bv + kb * pv_, pv_, im, csv);
                    h2[k] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(mag * trig, ev));
                }
                av[i / 2] = h2[0] | (h2[1] << 16);
            }
            floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(av), P, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(av), PL, d, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(d[r], vsc, acc[t][r] * alpha);
            __builtin_amdgcn_sched_barrier(0);   // keep each coordinate tile's reads next to its product
        }
    }
    float* pp = a.part + ((size_t)item * 16 + n) * D;
#pragma unroll
    for (int t = 0; t < T; ++t)
        *reinterpret_cast<floatx4*>(pp + 16 * t + 4 * g) = acc[t];
    if (g == 0) *reinterpret_cast<float2*>(a.ml + ((size_t)item * 16 + n) * 2) = float2{m, l};
}

// one block of D threads per output row (b, h): merge the splits, apply the inverse real DFT
template <int D>
__global__ __launch_bounds__(D) void fmag_attn_combine_kernel(FmAttnArgs a) {
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
        acc = acc / L;
    }
    y[k] = acc;
    __syncthreads();
    const float* G = a.tv.G32 + (size_t)k * D;
    float o = 0.0f;
    for (int c = 0; c < D; ++c) o = fmaf(G[c], y[c], o);
    const size_t oi = (size_t)row * D + k;
    if (a.out_bf16) static_cast<__bf16*>(a.out)[oi] = (__bf16)o;
    else static_cast<float*>(a.out)[oi] = o;
}

template <int D, int RWM, bool PQK, bool PQV>
static hipError_t launch_fattn(const FmAttnArgs& a, hipStream_t s) {
    const size_t lds = 4096 + (size_t)(kFaThreads / 64) * 16 * D * 2 +
                       (size_t)(kFaThreads / 64) * (32 * (a.tk.rec_words + a.tv.rec_words) + 4) * 4;
    const void* kern = reinterpret_cast<const void*>(&fmag_attn_kernel<D, RWM, PQK, PQV>);
    if (lds > 65536) {
        const hipError_t e = allow_lds(kern);
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((a.n_streams * a.n_split + kFaThreads / 64 - 1) / (kFaThreads / 64));
    hipLaunchKernelGGL((fmag_attn_kernel<D, RWM, PQK, PQV>), dim3(blocks), dim3(kFaThreads), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned rows = (unsigned)(a.n_streams / a.hkv * a.hq);
    hipLaunchKernelGGL((fmag_attn_combine_kernel<D>), dim3(rows), dim3(D), 0, s, a);
    return hipGetLastError();
}

template <int D, int RWM>
static hipError_t launch_fattn_pq(const FmAttnArgs& a, hipStream_t s) {
    const bool qk = a.tk.p <= 8, qv = a.tv.p <= 8;
    if (qk) return qv ? launch_fattn<D, RWM, true, true>(a, s) : launch_fattn<D, RWM, true, false>(a, s);
    return qv ? launch_fattn<D, RWM, false, true>(a, s) : launch_fattn<D, RWM, false, false>(a, s);
}

// records of up to 28 words (b + p <= 12 at d = 128, every width at d = 64) take the smaller
// register prefetch; the larger covers 8-bit magnitudes with bf16 phases at d = 128 (51 words)
hipError_t launch_fmag_attention(const FmAttnArgs& a, hipStream_t s) {
    const int rw = max(a.tk.rec_words, a.tv.rec_words);
    if (a.tk.d == 64) return launch_fattn_pq<64, 28>(a, s);
    return rw <= 28 ? launch_fattn_pq<128, 28>(a, s) : launch_fattn_pq<128, 51>(a, s);
}

}  // namespace tq
