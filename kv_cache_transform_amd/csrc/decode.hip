// Decode kernel: x̂ = n16 · s ⊙ (H c[idx]) / sqrt(d), the inverse rotation of the encoder
// ("Ablation, Statistical Inference, and Validation for KV-Cache Compression", §2 TurboQuant).
// One wave64 = 16 vectors x 4 parts; part g reads its contiguous C·b/8 packed bytes, dequantises
// P coordinates per LDS lookup (P·b-bit field -> P centroids), runs the Hadamard network of
// common.hpp and writes runs of d/16 coordinates.
#include "common.hpp"
#include "kernels.hpp"

namespace tq {

__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

template <int D, int B, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int C = D / 4, R = D / 16;
    constexpr int P = lut_group_c(B), NE = 1 << (P * B);
    constexpr int NW = (C * B + 31) / 32;
    constexpr int CB = C * B / 8;
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);

    __shared__ float lut[NE * P];
    for (int i = threadIdx.x; i < NE * P; i += blockDim.x) lut[i] = a.t.lut_f32[i];
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int v = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
    // block = one stream's tile range; waves take every 4th tile
    const int64_t st = blockIdx.x / a.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int head = (int)(st % a.t.n_heads);
    uint32_t smask[C];
    {
        const float* ss = a.t.signs_slot + ((int64_t)head * 4 + g) * C;
#pragma unroll
        for (int s = 0; s < C; ++s) smask[s] = f2u(ss[s]) & 0x80000000u;
    }
    const uint8_t* pidx = a.packed + a.off_idx + st * a.n_tokens * (int64_t)(D * B / 8) + g * CB;
    const uint16_t* pnrm = reinterpret_cast<const uint16_t*>(a.packed + a.off_norm) + st * a.n_tokens;
    // packed words and norm of one tile for this lane (zeros past the end)
    auto load_tile = [&](uint32_t (&w)[NW], uint32_t& nb, int64_t tl) {
        const int64_t tok = tl * 16 + v;
        if (tl < tb1 && tok < a.n_tokens) {
            load_bytes<CB, CA>(pidx + tok * (D * B / 8), w);
            nb = pnrm[tok];
        } else {
#pragma unroll
            for (int k = 0; k < NW; ++k) w[k] = 0u;
            nb = 0u;
        }
    };
    uint32_t wn[NW], nbn;
    load_tile(wn, nbn, tb0 + wave);
#pragma unroll 1
    for (int64_t tile = tb0 + wave; tile < tb1; tile += 4) {
        const int64_t tok = tile * 16 + v;
        const bool valid = tok < a.n_tokens;
        const int64_t vec = st * a.n_tokens + (valid ? tok : 0);
        uint32_t w[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = wn[k];
        const float nrm = (float)__builtin_bit_cast(_Float16, (uint16_t)nbn);
        load_tile(wn, nbn, tile + 4);       // next tile's loads overlap this tile's math
        float x[C];
#pragma unroll
        for (int q = 0; q < C / P; ++q) {
            const uint32_t f = get_bits<P * B>(w, q * P * B);
            const float* e = lut + f * P;
#pragma unroll
            for (int k = 0; k < P; ++k) x[q * P + k] = e[k];
        }
        fwht_slots<C, 1>(x);
        fwht_cross<C>(x);
        const float sc = nrm * kInvSqrtD;
        if (!valid) continue;
        if constexpr (OUT_BF16) {
            uint8_t* base = reinterpret_cast<uint8_t*>(a.out) + vec * (int64_t)(2 * D) + 2 * g * R;
            constexpr int RB = 2 * R;
            constexpr int RA = cmin(pow2_align(RB), 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t o[R / 2];
#pragma unroll
                for (int k = 0; k < R / 2; ++k) {
                    const int s0 = r * R + 2 * k;
                    o[k] = bf16_pair_rne(u2f(f2u(x[s0] * sc) ^ smask[s0]), u2f(f2u(x[s0 + 1] * sc) ^ smask[s0 + 1]));
                }
                store_bytes<RB, RA>(base + r * (D / 2), o);
            }
        } else {
            uint8_t* base = reinterpret_cast<uint8_t*>(a.out) + vec * (int64_t)(4 * D) + 4 * g * R;
            constexpr int RB = 4 * R;
            constexpr int RA = cmin(pow2_align(RB), 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t o[R];
#pragma unroll
                for (int k = 0; k < R; ++k) o[k] = f2u(x[r * R + k] * sc) ^ smask[r * R + k];
                store_bytes<RB, RA>(base + r * D, o);
            }
        }
    }
}

template <int D, int B, bool BF>
static hipError_t launch_one(const DecodeArgs& a, int num_cus, hipStream_t s) {
    DecodeArgs b = a;
    const int64_t target = (int64_t)num_cus * 4;
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    hipLaunchKernelGGL((decode_kernel<D, B, BF>), dim3((unsigned)(a.n_streams * bps)), dim3(256), 0, s, b);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, bool bf, int num_cus, hipStream_t s) {
#define TQ_DEC_CASE(BB) \
    case BB: return bf ? launch_one<D, BB, true>(a, num_cus, s) : launch_one<D, BB, false>(a, num_cus, s);
    switch (a.t.b) {
        TQ_DEC_CASE(1) TQ_DEC_CASE(2) TQ_DEC_CASE(3) TQ_DEC_CASE(4)
        TQ_DEC_CASE(5) TQ_DEC_CASE(6) TQ_DEC_CASE(7) TQ_DEC_CASE(8)
    }
#undef TQ_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s) {
    switch (a.t.d) {
        case 64: return launch_d<64>(a, out_bf16, num_cus, s);
        case 128: return launch_d<128>(a, out_bf16, num_cus, s);
        case 256: return launch_d<256>(a, out_bf16, num_cus, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
