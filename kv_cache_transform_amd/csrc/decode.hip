// Decode kernel: x̂ = n16 · s ⊙ (H c[idx]) / sqrt(d), the inverse rotation of the encoder
// ("Ablation, Statistical Inference, and Validation for KV-Cache Compression", §2 TurboQuant).
// One wave64 = 16 vectors x 4 parts; part g reads its contiguous C·b/8 packed bytes (coordinates
// g C .. g C + C - 1).  The Hadamard transform is split as in the encoder: the 32-point block over
// the index bits {0,1,2, n-2, n-1} runs on v_mfma_f32_16x16x32_f16 with the ±1 matrix as A and the
// dequantised centroids as B, given as fp16 hi + lo parts of 2^12 c (two products, fp32 accumulation,
// centroids to 2^-22 relative; the power-of-two scale keeps lo normal and is undone with the norm),
// and the middle bits are radix-2 butterflies in registers.  The
// output of part g is again coordinates g C .. g C + C - 1, scaled by n16/sqrt(d) with the signs.
#include <map>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace tq {

__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

template <int D, int B, bool OUT_BF16>
__global__ __launch_bounds__(256, (D == 256 && B == 6 && !OUT_BF16) ? 1 : 2) void decode_kernel(DecodeArgs a) {
    constexpr int C = D / 4, NKB = D / 32;
    constexpr int P = lut_group_c(B), NE = 1 << (P * B);
    constexpr int NW = (C * B + 31) / 32;
    constexpr int CB = C * B / 8;
    constexpr int CA = cmin(pow2_align(CB), 16);
    constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);

    // entry f: P hi halves then P lo halves of the P centroids of the P·b-bit field f
    __shared__ __align__(16) _Float16 lut[NE * P * 2];
    constexpr int ES = OUT_BF16 ? 2 : 4;
    constexpr int ROW = ES * D;                          // output bytes per vector
    constexpr int ROWP = ROW + 16;                       // padded LDS row
    constexpr int STG = 16 * ROWP;                       // LDS staging bytes per wave
    __shared__ __align__(16) uint8_t stage[4 * STG];
    for (int i = threadIdx.x; i < NE * P * 2; i += blockDim.x) lut[i] = a.t.lut_hl[i];
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
    // ±1 A tiles of the 32-point block (row 4 mg + mi = lane % 16, columns 8 g + jj): output bits
    // {n-2,n-1} = mg, bit 2 = h, bits {0,1} = mi; input bits {n-2,n-1} = g, bits {0,1,2} = jj
    half8 A0[2];
    {
        const int mi = lane & 3, mg = (lane >> 2) & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 wv;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t w2 = 0u;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int jj = 2 * t + q;
                    const uint32_t par = (uint32_t)(__builtin_popcount(mi & jj & 3) + h * (jj >> 2) +
                                                    __builtin_popcount(mg & g)) & 1u;
                    w2 |= (0x3c00u | (par << 15)) << (16 * q);
                }
                wv[t] = w2;
            }
            A0[h] = __builtin_bit_cast(half8, wv);
        }
    }
    uint32_t smask[C];       // sign bit of output coordinate g C + s
    {
        const float* ss = a.t.signs + (int64_t)head * D + g * C;
#pragma unroll
        for (int s = 0; s < C; ++s) smask[s] = f2u(ss[s]) & 0x80000000u;
    }
    const uint8_t* pidx = a.packed + a.off_idx + st * a.n_tokens * (int64_t)(D * B / 8) + g * CB;
    const uint16_t* pnrm = reinterpret_cast<const uint16_t*>(a.packed + a.off_norm) + st * a.n_tokens;
    // packed words and norm of one tile for this lane (a vector past the end reads token 0 of the
    // stream: in bounds, never stored)
    auto load_tile = [&](uint32_t (&w)[NW], uint32_t& nb, int64_t tl) {
        const int64_t tok = tl * 16 + v;
        const int64_t tk = tok < a.n_tokens ? tok : 0;
        load_bytes<CB, CA>(pidx + tk * (D * B / 8), w);
        nb = pnrm[tk];
    };
    uint32_t wn[NW], nbn;
    if (tb0 + wave < tb1) load_tile(wn, nbn, tb0 + wave);
#pragma unroll 1
    for (int64_t tile = tb0 + wave; tile < tb1; tile += 4) {
        uint32_t w[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = wn[k];
        const float nrm = (float)__builtin_bit_cast(_Float16, (uint16_t)nbn);
        if (tile + 4 < tb1) load_tile(wn, nbn, tile + 4);   // next tile's loads overlap this tile's math
        float x[C];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            // B operands: the 8 coordinates g C + 8 kb + jj, as fp16 hi and lo parts
            half8 bh, bl;
#pragma unroll
            for (int q = 0; q < 8 / P; ++q) {
                const uint32_t f = get_bits<P * B>(w, (8 * kb + q * P) * B);
                const _Float16* e = lut + f * (2 * P);
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    bh[q * P + k] = e[k];
                    bl[q * P + k] = e[P + k];
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[h], bh, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[h], bl, r, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) x[8 * kb + 4 * h + i] = r[i];
            }
        }
        fwht_slots<C, 8>(x);
        const float sc = nrm * (kInvSqrtD / 4096.0f);     // the LUT holds 2^12 c
        // the wave's 16 vectors are 16 consecutive rows of the output, one contiguous 16 ES d-byte
        // block: stage the rows in LDS (row stride padded by 16 bytes against bank conflicts) and
        // write the block back linearly, 1 KiB per store instruction
        constexpr int NOW = OUT_BF16 ? C / 2 : C;      // output words per lane
        uint32_t o[NOW];
        if constexpr (OUT_BF16) {
#pragma unroll
            for (int k = 0; k < C / 2; ++k)
                o[k] = bf16_pair_rne(u2f(f2u(x[2 * k] * sc) ^ smask[2 * k]), u2f(f2u(x[2 * k + 1] * sc) ^ smask[2 * k + 1]));
        } else {
#pragma unroll
            for (int k = 0; k < C; ++k) o[k] = f2u(x[k] * sc) ^ smask[k];
        }
        uint8_t* wst = stage + wave * STG;
#pragma unroll
        for (int k = 0; k < NOW / 4; ++k)
            *reinterpret_cast<u32x4*>(wst + v * ROWP + g * (4 * NOW) + 16 * k) =
                u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
        __builtin_amdgcn_wave_barrier();
        const int64_t nvalid = a.n_tokens - tile * 16;   // rows of this tile inside the stream
        uint8_t* gdst = reinterpret_cast<uint8_t*>(a.out) + (st * a.n_tokens + tile * 16) * (int64_t)ROW;
#pragma unroll
        for (int r = 0; r < ROW / 64; ++r) {
            const int off = r * 1024 + 16 * lane;      // linear byte offset within the block
            const int row = off / ROW, col = off - row * ROW;
            const u32x4 val = *reinterpret_cast<const u32x4*>(wst + row * ROWP + col);
            if (row < nvalid) *reinterpret_cast<u32x4*>(gdst + off) = val;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// resident blocks per CU of kernel k (cached per kernel)
static int decode_blocks_per_cu(const void* k) {
    static std::mutex mu;
    static std::map<const void*, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(k);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 256, 0) != hipSuccess || n < 1) n = 1;
    cache[k] = n;
    return n;
}

template <int D, int B, bool BF>
static hipError_t launch_one(const DecodeArgs& a, int num_cus, hipStream_t s) {
    DecodeArgs b = a;
    const int64_t target = (int64_t)num_cus * decode_blocks_per_cu(reinterpret_cast<const void*>(&decode_kernel<D, B, BF>));
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
