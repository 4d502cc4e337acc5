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
    const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    int64_t tile = wave_id * a.tiles_per_wave;
    const int64_t tile_end = tile + a.tiles_per_wave < a.n_tiles ? tile + a.tiles_per_wave : a.n_tiles;

    int cur_head = -1;
    uint32_t smask[C];
    for (; tile < tile_end; ++tile) {
        const int64_t st = tile / a.tiles_per_stream;
        const int64_t tok = (tile - st * a.tiles_per_stream) * 16 + v;
        const bool valid = tok < a.n_tokens;
        const int head = (int)(st % a.t.n_heads);
        if (head != cur_head) {
            cur_head = head;
            const float* ss = a.t.signs_slot + ((int64_t)head * 4 + g) * C;
#pragma unroll
            for (int s = 0; s < C; ++s) smask[s] = f2u(ss[s]) & 0x80000000u;
        }
        const int64_t vec = st * a.n_tokens + (valid ? tok : 0);
        uint32_t w[NW];
        float nrm = 0.0f;
        if (valid) {
            load_bytes<CB, CA>(a.packed + a.off_idx + vec * (int64_t)(D * B / 8) + g * CB, w);
            nrm = (float)*reinterpret_cast<const _Float16*>(a.packed + a.off_norm + vec * 2);
        } else {
#pragma unroll
            for (int k = 0; k < NW; ++k) w[k] = 0u;
        }
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
    const int64_t max_waves = (int64_t)num_cus * 16;
    const int64_t waves = a.n_tiles < max_waves ? a.n_tiles : max_waves;
    const int64_t blocks = (waves + 3) / 4;
    DecodeArgs b = a;
    b.tiles_per_wave = (a.n_tiles + blocks * 4 - 1) / (blocks * 4);
    hipLaunchKernelGGL((decode_kernel<D, B, BF>), dim3((unsigned)blocks), dim3(256), 0, s, b);
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
