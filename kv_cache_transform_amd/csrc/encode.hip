// Encode kernel ("Ablation, Statistical Inference, and Validation for KV-Cache Compression",
// §2 TurboQuant): per vector x, n = ||x||, y = H (x ⊙ s) / (sqrt(d) n), idx_j = #{i : t_i <= y_j},
// b-bit packing; with m > 0 also e = y - c[idx], ||e|| and sign(S e) (1-bit QJL of the residual).
//
// Work split: one wave64 = 16 vectors x 4 parts (see common.hpp).  Waves walk a contiguous range of
// 16-vector tiles, so the per-head sign constants are reloaded only when the stream changes.
// Search: a uniform grid over y in [-1,1] held in LDS maps y to the one threshold that can lie in
// its cell plus the count of thresholds below; one compare finishes the search for any b.
// S·e: v_mfma_f32_16x16x32_f16 with the lane's own residual as the B operand (lane l = vector
// l%16, k-block l/16 matches the MFMA operand layout), e split into fp16 hi + lo parts (prescaled
// by 2^14, |e| 2^14 < 2^15 always), S stored as fp16 values; accumulation in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace tq {

template <int D, int B, bool QJL, bool BF16, bool S_LDS>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
    constexpr int C = D / 4, R = D / 16, L = 1 << B;
    constexpr int NW = (C * B + 31) / 32;          // packed words per lane
    constexpr int CB = C * B / 8;                   // packed bytes per lane
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);
    constexpr int NG = (QJL && D <= 128) ? 2 : 1;   // 16-vector groups per pass (S-tile reuse)
    constexpr int SP = D + 8;                       // padded LDS row of S (halves)

    // ---- block = one stream's tile range; the RNG head is block-uniform -----------------------
    const int64_t st = blockIdx.x / a.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int m = a.t.m;

    extern __shared__ uint32_t lds[];
    const int G = a.t.G;
    const int ngw = 2 * (G + 3);
    for (int i = threadIdx.x; i < ngw; i += blockDim.x) lds[i] = a.t.grid[i];
    float* lds_c = reinterpret_cast<float*>(lds + ngw);
    _Float16* lds_S = reinterpret_cast<_Float16*>(lds + ngw + L + ((ngw + L) & 3 ? 4 - ((ngw + L) & 3) : 0));
    if constexpr (QJL) {
        for (int i = threadIdx.x; i < L; i += blockDim.x) lds_c[i] = a.t.cent_x1024[i];
        if constexpr (S_LDS) {
            const u32x4* src = reinterpret_cast<const u32x4*>(a.t.S + (int64_t)head * m * D);
            const int n16 = m * D / 8;             // 16-byte pieces
            for (int i = threadIdx.x; i < n16; i += blockDim.x) {
                const int row = i / (D / 8), col = i - row * (D / 8);
                *reinterpret_cast<u32x4*>(lds_S + row * SP + col * 8) = src[i];
            }
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int v = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const float gA = 0.5f * (float)G;
    const float gB = 0.5f * (float)G + 1.0f;       // entry 0 is a guard cell

    uint32_t Ps[BF16 ? C / 2 : 1];
    float sg[BF16 ? 1 : C];
    {
        const float* ss = a.t.signs_slot + ((int64_t)head * 4 + g) * C;
        if constexpr (BF16) {
#pragma unroll
            for (int k = 0; k < C / 2; ++k) Ps[k] = (f2u(ss[2 * k]) >> 16) | (f2u(ss[2 * k + 1]) & 0xffff0000u);
        } else {
#pragma unroll
            for (int s = 0; s < C; ++s) sg[s] = ss[s];
        }
    }
    // QJL A-operand rows: MFMA row slot rho of tile tau is sketch row (rho/4)*(m/4) + 4 tau + rho%4,
    // so lane part g collects rows [g m/4, (g+1) m/4), a contiguous bit chunk of the sketch.
    const int rho = lane & 15;
    const int row_base = (rho >> 2) * (m >> 2) + (rho & 3);

    // raw input words of one 16-vector group (runs of R coordinates, see common.hpp)
    constexpr int NIW = BF16 ? C / 2 : C;
    auto load_group = [&](uint32_t (&w)[NIW], int64_t tile) {
        const int64_t tok = tile * 16 + v;
        const bool valid = tile < tb1 && tok < a.n_tokens;
        const int64_t vec = st * a.n_tokens + (valid ? tok : 0);
        constexpr int ES = BF16 ? 2 : 4;              // element size
        constexpr int RB = ES * R;                    // bytes per run
        constexpr int RA = cmin(pow2_align(RB), 16);
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x) + vec * (int64_t)(ES * D) + ES * g * R;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (valid) load_bytes<RB, RA>(base + r * (ES * D / 4), &w[r * (NIW / 4)]);
            else {
#pragma unroll
                for (int k = 0; k < NIW / 4; ++k) w[r * (NIW / 4) + k] = 0u;
            }
        }
    };
    uint32_t nxt[NG][NIW];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) load_group(nxt[gi], tb0 + wave * NG + gi);

#pragma unroll 1
    for (int64_t t = tb0 + wave * NG; t < tb1; t += 4 * NG) {
        uint32_t cur[NG][NIW];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int k = 0; k < NIW; ++k) cur[gi][k] = nxt[gi][k];
        if (t + 4 * NG < tb1) {            // issue the next pass's loads before this pass's math
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) load_group(nxt[gi], t + 4 * NG + gi);
        }
        half8 bh[NG][QJL ? C / 8 : 1], bl[NG][QJL ? C / 8 : 1];
        float e2v[NG];
        bool validv[NG];
        int64_t vecv[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int64_t tok = (t + gi) * 16 + v;
            const bool valid = (t + gi) < tb1 && tok < a.n_tokens;
            const int64_t vec = st * a.n_tokens + (valid ? tok : 0);
            validv[gi] = valid;
            vecv[gi] = vec;

            // ---- sign, first butterfly stage, norm ----------------------------------------------
            float x[C];
            float n2 = 0.0f;
            const uint32_t (&w)[NIW] = cur[gi];
            if constexpr (BF16) {
#pragma unroll
                for (int k = 0; k < C / 2; ++k) {
                    const bf16x2 wv = __builtin_bit_cast(bf16x2, w[k]);
                    x[2 * k] = dot2_bf16(w[k], Ps[k]);          // s_i x_i + s_{i+1} x_{i+1}
                    x[2 * k + 1] = dot2_bf16_nhi(w[k], Ps[k]);  // s_i x_i - s_{i+1} x_{i+1}
                    n2 = __builtin_amdgcn_fdot2_f32_bf16(wv, wv, n2, false);
                }
                fwht_slots<C, 2>(x);
            } else {
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
            const float sA = sc * gA;

            // ---- scalar quantiser + pack (and the scaled residual for QJL) ----------------------
            // The grid lives in the affine domain u = y G/2 + G/2 + 1; thresholds are stored there.
            uint32_t pk[NW];
#pragma unroll
            for (int k = 0; k < NW; ++k) pk[k] = 0u;
            float e2 = 0.0f;
#pragma unroll
            for (int s = 0; s < C; ++s) {
                float y, u;
                if constexpr (QJL) {
                    y = x[s] * sc;
                    u = fmaf(y, gA, gB);
                } else {
                    u = fmaf(x[s], sA, gB);
                }
                const uint32_t cell = (uint32_t)u;
                const uint32_t thr = lds[2 * cell], base = lds[2 * cell + 1];
                const uint32_t idx = base + (u >= u2f(thr) ? 1u : 0u);
                put_bits<B>(pk, s * B, idx);
                if constexpr (QJL) {
                    const float e = fmaf(y, 16384.0f, -lds_c[idx]);  // 2^14 (y - c[idx])
                    x[s] = e;
                    e2 = fmaf(e, e, e2);
                }
            }
            if (valid) {
                store_bytes<CB, CA>(a.packed + a.off_idx + vec * (int64_t)(D * B / 8) + g * CB, pk);
                if (g == 0) *reinterpret_cast<_Float16*>(a.packed + a.off_norm + vec * 2) = (_Float16)n;
            }
            if constexpr (QJL) {
                e2v[gi] = e2;
                // B operands: lane's residual slots [8k, 8k+8) for k-step k, exact hi + lo split
#pragma unroll
                for (int k = 0; k < C / 8; ++k) {
                    u32x4 hv, lv;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float e0 = x[8 * k + 2 * u], e1 = x[8 * k + 2 * u + 1];
                        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
                        hv[u] = h;
                        lv[u] = sub_f16pair_from_f32(h, e0, e1);
                    }
                    bh[gi][k] = __builtin_bit_cast(half8, hv);
                    bl[gi][k] = __builtin_bit_cast(half8, lv);
                }
            }
        }

        if constexpr (QJL) {
            const _Float16* Sg = S_LDS ? (lds_S + g * C) : (a.t.S + (int64_t)head * m * D + g * C);
            const int rs = S_LDS ? SP : D;
            // sketch bits of lane part g: rows [g m/4, (g+1) m/4), 32 per word; within a word the
            // 8 tiles are visited in descending order and each z shifts its sign bit in at bit 0
            // (alignbit), so bit p ends up holding row p; the word is inverted at the end (z >= 0).
            const int nbits = m >> 2;
            for (int wb = 0; wb < nbits; wb += 32) {
                const int nt = (nbits - wb) >= 32 ? 8 : ((nbits - wb) >> 2);
                uint32_t bits[NG];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) bits[gi] = 0u;
#pragma unroll
                for (int tt = 7; tt >= 0; --tt) {
                    if (tt < nt) {
                        const int tau = (wb >> 2) + tt;
                        floatx4 acc[NG];
#pragma unroll
                        for (int gi = 0; gi < NG; ++gi) acc[gi] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                        const _Float16* Srow = Sg + (row_base + 4 * tau) * rs;
#pragma unroll
                        for (int k = 0; k < C / 8; ++k) {
                            const half8 A = *reinterpret_cast<const half8*>(Srow + 8 * k);
#pragma unroll
                            for (int gi = 0; gi < NG; ++gi) {
                                acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[gi][k], acc[gi], 0, 0, 0);
                                acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[gi][k], acc[gi], 0, 0, 0);
                            }
                        }
#pragma unroll
                        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                            for (int i = 3; i >= 0; --i) bits[gi] = __builtin_amdgcn_alignbit(bits[gi], f2u(acc[gi][i]), 31);
                    }
                }
                const int nb = nt >> 1;                       // bytes in this word
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    if (validv[gi]) {
                        const uint32_t bw = ~bits[gi];
                        uint8_t* dst = a.packed + a.off_sketch + vecv[gi] * (int64_t)(m / 8) + g * (m / 32) + (wb >> 3);
                        if (nb == 4 && (m & 127) == 0) *reinterpret_cast<uint32_t*>(dst) = bw;
                        else if (nb == 2 && (m & 63) == 0) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bw;
                        else for (int q = 0; q < nb; ++q) dst[q] = (uint8_t)(bw >> (8 * q));
                    }
                }
            }
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const float e2 = sum4(e2v[gi]);
                if (validv[gi] && g == 0)
                    *reinterpret_cast<_Float16*>(a.packed + a.off_rnorm + vecv[gi] * 2) =
                        (_Float16)(sqrtf(e2) * (1.0f / 16384.0f));
            }
        }
    }
}

template <int D, int B, bool QJL, bool BF16>
static hipError_t launch_one(const EncodeArgs& a, int num_cus, hipStream_t s) {
    EncodeArgs b = a;
    const int64_t target = (int64_t)num_cus * 4;
    int64_t bps = (target + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    const int L = 1 << B;
    const size_t head_bytes = (size_t)(2 * (a.t.G + 3) + L + 4) * 4;
    const size_t s_bytes = (size_t)a.t.m * (D + 8) * 2;
    const bool s_lds = QJL && s_bytes <= 65536;
    const size_t lds = head_bytes + (s_lds ? s_bytes : 0);
    const dim3 grid((unsigned)(a.n_streams * bps));
    if (s_lds) hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, true>), grid, dim3(256), lds, s, b);
    else hipLaunchKernelGGL((encode_kernel<D, B, QJL, BF16, false>), grid, dim3(256), lds, s, b);
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
