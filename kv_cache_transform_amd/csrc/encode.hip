// Encode kernel ("Ablation, Statistical Inference, and Validation for KV-Cache Compression",
// §2 TurboQuant): per vector x, n = ||x||, y = H (x ⊙ s) / (sqrt(d) n), idx_j = #{i : t_i <= y_j},
// b-bit packing; with m > 0 also e = y - c[idx], ||e|| and sign(S e) (1-bit QJL of the residual).
//
// Work split: one wave64 = 16 vectors x 4 parts (see common.hpp).  Waves walk a contiguous range of
// 16-vector tiles, so the per-head sign constants are reloaded only when the stream changes.
// Search: a uniform grid over y in [-1,1] held in LDS maps y to the one threshold that can lie in
// its cell plus the count of thresholds below; one compare finishes the search for any b.
// S·e: v_mfma_f32_16x16x32_f16 with the lane's own residual as the B operand (lane l = vector
// l%16, k-block l/16 matches the MFMA operand layout), e split exactly into fp16 hi + lo parts
// (prescaled by 2^10), S stored as fp16 values; accumulation in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace tq {

template <int D, int B, bool QJL, bool BF16>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
    constexpr int C = D / 4, R = D / 16, L = 1 << B;
    constexpr int NW = (C * B + 31) / 32;          // packed words per lane
    constexpr int CB = C * B / 8;                   // packed bytes per lane
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);

    extern __shared__ uint32_t lds[];
    const int G = a.t.G;
    const int ngw = 2 * (G + 3);
    for (int i = threadIdx.x; i < ngw; i += blockDim.x) lds[i] = a.t.grid[i];
    float* lds_c = reinterpret_cast<float*>(lds + ngw);
    if constexpr (QJL)
        for (int i = threadIdx.x; i < L; i += blockDim.x) lds_c[i] = a.t.cent_x1024[i];
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int v = lane & 15, g = lane >> 4;
    const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    int64_t tile = wave_id * a.tiles_per_wave;
    const int64_t tile_end = tile + a.tiles_per_wave < a.n_tiles ? tile + a.tiles_per_wave : a.n_tiles;
    const float gA = 0.5f * (float)G;
    const float gB = 0.5f * (float)G + 1.0f;       // entry 0 is a guard cell
    const int m = a.t.m;

    int cur_head = -1;
    uint32_t Ps[BF16 ? C / 2 : 1], Ms[BF16 ? C / 2 : 1];
    float sg[BF16 ? 1 : C];

    for (; tile < tile_end; ++tile) {
        const int64_t st = tile / a.tiles_per_stream;
        const int64_t tok = (tile - st * a.tiles_per_stream) * 16 + v;
        const bool valid = tok < a.n_tokens;
        const int head = (int)(st % a.t.n_heads);
        if (head != cur_head) {
            cur_head = head;
            const float* ss = a.t.signs_slot + ((int64_t)head * 4 + g) * C;
            if constexpr (BF16) {
#pragma unroll
                for (int k = 0; k < C / 2; ++k) {
                    Ps[k] = (f2u(ss[2 * k]) >> 16) | (f2u(ss[2 * k + 1]) & 0xffff0000u);
                    Ms[k] = Ps[k] ^ 0x80000000u;
                }
            } else {
#pragma unroll
                for (int s = 0; s < C; ++s) sg[s] = ss[s];
            }
        }
        const int64_t vec = st * a.n_tokens + (valid ? tok : 0);

        // ---- load, sign, first butterfly stage, norm ------------------------------------------
        float x[C];
        float n2 = 0.0f;
        if constexpr (BF16) {
            uint32_t w[C / 2];
            constexpr int RB = 2 * R;                  // bytes per run
            constexpr int RA = cmin(pow2_align(RB), 16);
            const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x) + vec * (int64_t)(2 * D) + 2 * g * R;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (valid) load_bytes<RB, RA>(base + r * (D / 2), &w[r * (R / 2)]);
                else {
#pragma unroll
                    for (int k = 0; k < R / 2; ++k) w[r * (R / 2) + k] = 0u;
                }
            }
#pragma unroll
            for (int k = 0; k < C / 2; ++k) {
                const bf16x2 wv = __builtin_bit_cast(bf16x2, w[k]);
                x[2 * k] = __builtin_amdgcn_fdot2_f32_bf16(wv, __builtin_bit_cast(bf16x2, Ps[k]), 0.0f, false);
                x[2 * k + 1] = __builtin_amdgcn_fdot2_f32_bf16(wv, __builtin_bit_cast(bf16x2, Ms[k]), 0.0f, false);
                n2 = __builtin_amdgcn_fdot2_f32_bf16(wv, wv, n2, false);
            }
            fwht_slots<C, 2>(x);
        } else {
            constexpr int RB = 4 * R;
            constexpr int RA = cmin(pow2_align(RB), 16);
            const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x) + vec * (int64_t)(4 * D) + 4 * g * R;
            uint32_t w[C];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (valid) load_bytes<RB, RA>(base + r * D, &w[r * R]);
                else {
#pragma unroll
                    for (int k = 0; k < R; ++k) w[r * R + k] = 0u;
                }
            }
#pragma unroll
            for (int s = 0; s < C; ++s) {
                const float xv = u2f(w[s]);
                n2 = fmaf(xv, xv, n2);
                x[s] = xv * sg[s];
            }
            fwht_slots<C, 1>(x);
        }
        fwht_cross<C>(x);
        n2 = sum4(n2);
        const float n = sqrtf(n2);
        const float sc = n > 0.0f ? kInvSqrtD / n : 0.0f;

        // ---- scalar quantiser + pack (and the scaled residual for QJL) ------------------------
        uint32_t pk[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) pk[k] = 0u;
        float e2 = 0.0f;
#pragma unroll
        for (int s = 0; s < C; ++s) {
            const float y = x[s] * sc;
            const uint32_t cell = (uint32_t)fmaf(y, gA, gB);
            const uint32_t thr = lds[2 * cell], base = lds[2 * cell + 1];
            const uint32_t idx = base + (y >= u2f(thr) ? 1u : 0u);
            put_bits<B>(pk, s * B, idx);
            if constexpr (QJL) {
                const float e = fmaf(y, 1024.0f, -lds_c[idx]);   // 2^10 (y - c[idx])
                x[s] = e;
                e2 = fmaf(e, e, e2);
            }
        }
        if (valid) {
            store_bytes<CB, CA>(a.packed + a.off_idx + vec * (int64_t)(D * B / 8) + g * CB, pk);
            if (g == 0) {
                const _Float16 h = (_Float16)n;
                *reinterpret_cast<_Float16*>(a.packed + a.off_norm + vec * 2) = h;
            }
        }

        if constexpr (QJL) {
            e2 = sum4(e2);
            // B operands: lane's residual slots [8k, 8k+8) for k-step k, exact hi + lo split
            half8 bh[C / 8], bl[C / 8];
#pragma unroll
            for (int k = 0; k < C / 8; ++k) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float e0 = x[8 * k + 2 * t], e1 = x[8 * k + 2 * t + 1];
                    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(e0, e1));
                    const half2v l = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(e0 - (float)h[0], e1 - (float)h[1]));
                    bh[k][2 * t] = h[0];
                    bh[k][2 * t + 1] = h[1];
                    bl[k][2 * t] = l[0];
                    bl[k][2 * t + 1] = l[1];
                }
            }
            // A operand rows: MFMA row slot rho = 4*(rho/4) + rho%4 of tile tau maps to sketch row
            // (rho/4)*(m/4) + 4*tau + rho%4, so lane part g ends up with rows [g*m/4, (g+1)*m/4).
            const int rho = lane & 15;
            const _Float16* Sh = a.t.S + (int64_t)cur_head * m * D + g * C;
            const int row_base = (rho >> 2) * (m >> 2) + (rho & 3);
            uint8_t* skp = a.packed + a.off_sketch + vec * (int64_t)(m / 8) + g * (m / 32);
            uint32_t bits = 0u;
            const int ntile = m >> 4;
            for (int tau = 0; tau < ntile; ++tau) {
                floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
                const _Float16* Srow = Sh + (int64_t)(row_base + 4 * tau) * D;
#pragma unroll
                for (int k = 0; k < C / 8; ++k) {
                    const half8 A = *reinterpret_cast<const half8*>(Srow + 8 * k);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[k], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[k], acc, 0, 0, 0);
                }
                const int pos = (4 * tau) & 31;
                bits |= (acc[0] >= 0.0f ? 1u : 0u) << pos;
                bits |= (acc[1] >= 0.0f ? 1u : 0u) << (pos + 1);
                bits |= (acc[2] >= 0.0f ? 1u : 0u) << (pos + 2);
                bits |= (acc[3] >= 0.0f ? 1u : 0u) << (pos + 3);
                const bool word_done = (pos == 28) || (tau == ntile - 1);
                if (word_done) {
                    if (valid) {
                        const int wbyte = ((4 * tau) >> 5) * 4;
                        const int nb = (4 * (tau + 1) - ((4 * tau) & ~31)) / 8;  // bytes filled in this word
                        uint8_t* dst = skp + wbyte;
                        if (nb == 4 && (m & 127) == 0) *reinterpret_cast<uint32_t*>(dst) = bits;
                        else if (nb == 2 && (m & 63) == 0) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bits;
                        else for (int q = 0; q < nb; ++q) dst[q] = (uint8_t)(bits >> (8 * q));
                    }
                    bits = 0u;
                }
            }
            if (valid && g == 0) {
                const _Float16 h = (_Float16)(sqrtf(e2) * (1.0f / 1024.0f));
                *reinterpret_cast<_Float16*>(a.packed + a.off_rnorm + vec * 2) = h;
            }
        }
    }
}

template <int D, int B, bool QJL, bool BF16>
static hipError_t launch_one(const EncodeArgs& a, int num_cus, hipStream_t s) {
    const int64_t max_waves = (int64_t)num_cus * 16;
    int64_t waves = a.n_tiles < max_waves ? a.n_tiles : max_waves;
    const int64_t blocks = (waves + 3) / 4;
    EncodeArgs b = a;
    b.tiles_per_wave = (a.n_tiles + blocks * 4 - 1) / (blocks * 4);
    const size_t lds = (size_t)(2 * (a.t.G + 3)) * 4 + (QJL ? (size_t)(1 << B) * 4 : 0);
    hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16>), dim3((unsigned)blocks), dim3(256), lds, s, b);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t launch_db(const EncodeArgs& a, bool bf16, int num_cus, hipStream_t s) {
    const bool qjl = a.t.m > 0;
    if (bf16) return qjl ? launch_one<D, B, true, true>(a, num_cus, s) : launch_one<D, B, false, true>(a, num_cus, s);
    return qjl ? launch_one<D, B, true, false>(a, num_cus, s) : launch_one<D, B, false, false>(a, num_cus, s);
}

template <int D>
static hipError_t launch_d(const EncodeArgs& a, bool bf16, int num_cus, hipStream_t s) {
    switch (a.t.b) {
        case 1: return launch_db<D, 1>(a, bf16, num_cus, s);
        case 2: return launch_db<D, 2>(a, bf16, num_cus, s);
        case 3: return launch_db<D, 3>(a, bf16, num_cus, s);
        case 4: return launch_db<D, 4>(a, bf16, num_cus, s);
        case 5: return launch_db<D, 5>(a, bf16, num_cus, s);
        case 6: return launch_db<D, 6>(a, bf16, num_cus, s);
        case 7: return launch_db<D, 7>(a, bf16, num_cus, s);
        case 8: return launch_db<D, 8>(a, bf16, num_cus, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_encode(const EncodeArgs& a, bool x_bf16, int num_cus, hipStream_t s) {
    switch (a.t.d) {
        case 64: return launch_d<64>(a, x_bf16, num_cus, s);
        case 128: return launch_d<128>(a, x_bf16, num_cus, s);
        case 256: return launch_d<256>(a, x_bf16, num_cus, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
