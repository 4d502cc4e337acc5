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

// QJL = true: the corrected reconstruction x̂ = n16 · s ⊙ H (c[idx] + Δŷ) / sqrt(d) with
// Δŷ = sqrt(pi/2)/m · r16 · S^T (2σ - 1) ("Ablation...", §2 TurboQuant: the sketch correction added
// at decode, here for either sketch matrix).  S^T (2σ - 1) runs on v_mfma_f32_16x16x32_f16 with
// A = S^T (fp16, staged in LDS in operand order; row r of tile t is coordinate (r/4) C + 4 t + r%4,
// so lane part g receives its own coordinates g C + 4 t + i) and B = the ±1 sketch signs (exact),
// giving exact fp32 sums; c + Δŷ is then split into fp16 hi + lo parts of 2^12 (c + Δŷ) as the B
// operands of the inverse transform.
// LEAN (the corrected decode where S^T fills most of LDS: d = 256, m = 256): a lookup of one
// coordinate per entry (2^b entries) and direct stores of each lane's contiguous output coordinates
// instead of the staged row block, so S^T and the tables fit in 133 KiB whatever b is.
template <int D, int B, bool OUT_BF16, bool QJL = false, bool LEAN = false>
__global__ __launch_bounds__(256, (D == 256 && B == 6 && !OUT_BF16) || QJL ? 1 : 2) void decode_kernel(DecodeArgs a) {
    static_assert(!LEAN || QJL, "the lean form serves the corrected decode");
    constexpr int NWAVES = 4;
    constexpr int C = D / 4, NKB = D / 32;
    constexpr int PG = lut_group_c(B);                   // coordinates per entry of the device table
    constexpr int P = LEAN ? 1 : PG, NE = 1 << (P * B);
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
    __shared__ __align__(16) uint8_t stage[LEAN ? 16 : NWAVES * STG];
    if constexpr (LEAN) {
        // entry i: 2^12 c[i] as hi, lo: the device table's entry whose other coordinates are index 0
        for (int i = threadIdx.x; i < NE; i += blockDim.x) {
            lut[2 * i] = a.t.lut_hl[i * 2 * PG];
            lut[2 * i + 1] = a.t.lut_hl[i * 2 * PG + PG];
        }
    } else {
        // 16-byte pieces (the table is a multiple of 8 halves for every b; the device table is 256-byte
        // aligned), so the copy waits on memory once per 4 KiB rather than per 512 bytes
        static_assert((NE * P * 2) % 8 == 0, "whole 16-byte pieces");
        const u32x4* src = reinterpret_cast<const u32x4*>(a.t.lut_hl);
        for (int i = threadIdx.x; i < NE * P * 2 / 8; i += blockDim.x) reinterpret_cast<u32x4*>(lut)[i] = src[i];
    }
    // block = one stream's tile range; waves take every NWAVES-th tile
    const int64_t st = blockIdx.x / a.blocks_per_stream;
    const int64_t sub = blockIdx.x - st * a.blocks_per_stream;
    const int64_t tb0 = sub * a.tiles_per_block;
    const int64_t tb1 = tb0 + a.tiles_per_block < a.tiles_per_stream ? tb0 + a.tiles_per_block : a.tiles_per_stream;
    const int head = (int)(st % a.t.n_heads);
    const int m = a.t.m;
    const int KSM = m >> 5;                             // k-steps of 32 sketch rows
    extern __shared__ u32x4 qlds[];                    // QJL: S^T pieces, then the byte -> ±1 table
    // randomized Hadamard sketch: S^T (2σ - 1) = s2 ⊙ H (2σ - 1), the decode's own 32-point block and
    // butterflies on the ±1 signs, so S^T is not staged
    const bool rht = QJL && a.t.sketch == 1;
    const int np = rht ? 0 : (C / 4) * KSM * 64;     // S^T pieces in LDS before the sign table
    if constexpr (QJL) {
        // piece (t KSM + ks) 64 + l of lane l = r + 16 kc: S[32 ks + 8 kc + jj][(r/4) C + 4 t + r%4],
        // jj = 0..7, as 8 fp16
        const uint16_t* Sh = reinterpret_cast<const uint16_t*>(a.t.S) + (int64_t)head * m * D;
        for (int i = threadIdx.x; i < np; i += blockDim.x) {
            const int l = i & 63, tk = i >> 6, t = tk / KSM, ks = tk - t * KSM;
            const int r = l & 15, kc = l >> 4;
            const int coord = (r >> 2) * C + 4 * t + (r & 3);
            const uint16_t* col = Sh + (int64_t)(32 * ks + 8 * kc) * D + coord;
            u32x4 pc;
#pragma unroll
            for (int q = 0; q < 4; ++q) pc[q] = (uint32_t)col[(2 * q) * D] | ((uint32_t)col[(2 * q + 1) * D] << 16);
            qlds[i] = pc;
        }
        // byte e -> 8 fp16 of 2 bit_jj(e) - 1
        for (int e = threadIdx.x; e < 256; e += blockDim.x) {
            u32x4 pc;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pc[q] = (((e >> (2 * q)) & 1) ? 0x3c00u : 0xbc00u) | ((((e >> (2 * q + 1)) & 1) ? 0x3c00u : 0xbc00u) << 16);
            qlds[np + e] = pc;
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int v = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
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
    const bool plain = a.t.rotation == 1;              // Plain-KV: no inverse rotation, no signs
    uint32_t smask[C];       // sign bit of output coordinate g C + s
    {
        const float* ss = a.t.signs + (int64_t)head * D + g * C;
#pragma unroll
        for (int s = 0; s < C; ++s) smask[s] = plain ? 0u : f2u(ss[s]) & 0x80000000u;
    }
    uint32_t s2mask[QJL ? C : 1];   // RHT: sign bit of s2 at coordinate g C + s
    if constexpr (QJL) {
        if (rht) {
            const float* ss = a.t.signs2 + (int64_t)head * D + g * C;
#pragma unroll
            for (int s = 0; s < C; ++s) s2mask[s] = f2u(ss[s]) & 0x80000000u;
        }
    }
    const uint8_t* pidx = a.packed + a.off_idx + st * a.n_tokens * (int64_t)(D * B / 8) + g * CB;
    const uint16_t* pnrm = reinterpret_cast<const uint16_t*>(a.packed + a.off_norm) + st * a.n_tokens;
    const uint8_t* psk = a.packed + a.off_sketch + st * a.n_tokens * (int64_t)(m / 8);
    const uint16_t* prn = reinterpret_cast<const uint16_t*>(a.packed + a.off_rnorm) + st * a.n_tokens;
    constexpr int NSW = QJL ? D / 32 : 1;               // sketch dwords per vector at most (m <= d)
    // packed words, norm (and with QJL the sketch dwords and residual norm) of one tile for this
    // lane (a vector past the end reads token 0 of the stream: in bounds, never stored)
    auto load_tile = [&](uint32_t (&w)[NW], uint32_t& nb, uint32_t (&sk)[NSW], uint32_t& rb, int64_t tl) {
        const int64_t tok = tl * 16 + v;
        const int64_t tk = tok < a.n_tokens ? tok : 0;
        load_bytes<CB, CA>(pidx + tk * (D * B / 8), w);
        nb = pnrm[tk];
        if constexpr (QJL) {
            const uint8_t* sb = psk + tk * (int64_t)(m / 8);
            if (rht) {      // the lane's own NKB bytes: sketch rows g C .. g C + C - 1
                load_bytes<NKB, NKB>(sb + g * NKB, sk);
            } else {
                const uint32_t* sp = reinterpret_cast<const uint32_t*>(sb);
#pragma unroll
                for (int k = 0; k < NSW; ++k) sk[k] = k < KSM ? sp[k] : 0u;
            }
            rb = prn[tk];
        }
    };
    uint32_t wn[NW], nbn, skn[NSW], rbn = 0u;
    if (tb0 + wave < tb1) load_tile(wn, nbn, skn, rbn, tb0 + wave);
#pragma unroll 1
    for (int64_t tile = tb0 + wave; tile < tb1; tile += NWAVES) {
        uint32_t w[NW], sk[NSW];
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = wn[k];
#pragma unroll
        for (int k = 0; k < NSW; ++k) sk[k] = skn[k];
        const float nrm = (float)__builtin_bit_cast(_Float16, (uint16_t)nbn);
        const float rn = (float)__builtin_bit_cast(_Float16, (uint16_t)rbn);
        if (tile + NWAVES < tb1) load_tile(wn, nbn, skn, rbn, tile + NWAVES);   // next tile's loads overlap this tile's math
        // QJL: dl[s] = (S^T (2σ - 1)) at coordinate g C + s, scaled by 2^12 sqrt(pi/2)/m r16
        float dl[QJL ? C : 1];
        if constexpr (QJL) {
          const float kq = rn * (1.2533141373155003f * 4096.0f) / (float)m;   // 2^12 sqrt(pi/2)/m r16
          if (rht) {
            // H b on the ±1 signs of coordinates g C + 8 kb + jj (byte g C/8 + kb of the sketch),
            // exact in fp16 and fp32; then s2 and the scale
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const half8 Bs = __builtin_bit_cast(half8, qlds[__builtin_amdgcn_ubfe(sk[kb >> 2], 8 * (kb & 3), 8)]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[h], Bs, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dl[8 * kb + 4 * h + i] = r[i];
                }
            }
            fwht_slots<C, 8>(dl);
#pragma unroll
            for (int s2 = 0; s2 < C; ++s2) dl[s2] = u2f(f2u(dl[s2]) ^ s2mask[s2]) * kq;
          } else {
            floatx4 acc[C / 4];
#pragma unroll
            for (int t = 0; t < C / 4; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < NSW; ++ks) {
                if (ks < KSM) {
                    const half8 Bs = __builtin_bit_cast(half8, qlds[np + __builtin_amdgcn_ubfe(sk[ks], 8 * g, 8)]);
#pragma unroll
                    for (int t = 0; t < C / 4; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qlds[(t * KSM + ks) * 64 + lane]),
                                                                        Bs, acc[t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < C / 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dl[4 * t + i] = acc[t][i] * kq;
          }
        }
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
            if constexpr (QJL) {
                // 2^12 (c + Δŷ), re-split exactly into fp16 hi + lo
                u32x4 hv, lv;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float t0 = ((float)bh[2 * q] + (float)bl[2 * q]) + dl[8 * kb + 2 * q];
                    const float t1 = ((float)bh[2 * q + 1] + (float)bl[2 * q + 1]) + dl[8 * kb + 2 * q + 1];
                    const half2v hh = {(_Float16)t0, (_Float16)t1};
                    hv[q] = __builtin_bit_cast(uint32_t, hh);
                    lv[q] = sub_f16pair_from_f32(hv[q], t0, t1);
                }
                bh = __builtin_bit_cast(half8, hv);
                bl = __builtin_bit_cast(half8, lv);
            }
            if (plain) {                                   // no rotation: the coordinates themselves
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) x[8 * kb + jj] = (float)bh[jj] + (float)bl[jj];
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    floatx4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[h], bh, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    r = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[h], bl, r, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[8 * kb + 4 * h + i] = r[i];
                }
            }
        }
        if (!plain) fwht_slots<C, 8>(x);
        const float sc = nrm * ((plain ? 1.0f : kInvSqrtD) / 4096.0f);     // the LUT holds 2^12 c
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
        if constexpr (LEAN) {
            // the lane's coordinates g C .. g C + C - 1 of vector `tok` are ES·C contiguous bytes
            const int64_t tok = tile * 16 + v;
            if (tok < a.n_tokens) {
                uint8_t* dst = reinterpret_cast<uint8_t*>(a.out) + (st * a.n_tokens + tok) * (int64_t)ROW + g * (4 * NOW);
#pragma unroll
                for (int k = 0; k < NOW / 4; ++k)
                    *reinterpret_cast<u32x4*>(dst + 16 * k) = u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
            }
        } else {
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

// raise kernel k's dynamic LDS limit to `bytes` once
static hipError_t raise_dyn_lds(const void* k, int bytes) {
    static std::mutex mu;
    static std::map<const void*, int> done;
    std::lock_guard<std::mutex> lock(mu);
    auto it = done.find(k);
    if (it != done.end() && it->second >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done[k] = bytes;
    return e;
}

// QJL-corrected decode: S^T in LDS (d m 2 bytes) plus the 4 KiB sign table as dynamic LDS beside the
// kernel's static LUT and staging buffer.  At d = 256 where that exceeds one CU's 160 KiB (m = 256),
// the lean form (no staging buffer, a 2^b-entry lookup) runs instead.
template <int D, int B, bool BF, bool LEAN>
static hipError_t launch_qjl_form(const DecodeArgs& a, int num_cus, hipStream_t s, size_t stat, size_t dyn) {
    constexpr size_t kLdsMax = 163840;
    constexpr int threads = 256;
    const void* kern = reinterpret_cast<const void*>(&decode_kernel<D, B, BF, true, LEAN>);
    if (dyn > 65536) {
        const hipError_t e = raise_dyn_lds(kern, (int)(kLdsMax - stat));
        if (e != hipSuccess) return e;
    }
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, dyn) != hipSuccess || nb < 1) nb = 1;
    DecodeArgs b = a;
    int64_t bps = ((int64_t)num_cus * nb + a.n_streams - 1) / a.n_streams;
    if (bps > a.tiles_per_stream) bps = a.tiles_per_stream;
    if (bps < 1) bps = 1;
    b.blocks_per_stream = bps;
    b.tiles_per_block = (a.tiles_per_stream + bps - 1) / bps;
    hipLaunchKernelGGL((decode_kernel<D, B, BF, true, LEAN>), dim3((unsigned)(a.n_streams * bps)), dim3(threads), dyn, s, b);
    return hipGetLastError();
}

template <int D, int B, bool BF>
static hipError_t launch_one_qjl(const DecodeArgs& a, int num_cus, hipStream_t s, bool* supported) {
    constexpr int P = lut_group_c(B), NE = 1 << (P * B);
    constexpr size_t kLdsMax = 163840;
    const size_t stat = (size_t)NE * P * 4 + (size_t)4 * 16 * ((BF ? 2 : 4) * D + 16);
    const size_t dyn = (a.t.sketch == 1 ? 0 : (size_t)D * a.t.m * 2) + 256 * 16;
    *supported = true;
    if (stat + dyn <= kLdsMax) return launch_qjl_form<D, B, BF, false>(a, num_cus, s, stat, dyn);
    if constexpr (D == 256) {
        const size_t lean = (size_t)(1 << B) * 4 + 16;
        if (lean + dyn <= kLdsMax) return launch_qjl_form<D, B, BF, true>(a, num_cus, s, lean, dyn);
    }
    *supported = false;
    return hipSuccess;
}

template <int D>
static hipError_t launch_d_qjl(const DecodeArgs& a, bool bf, int num_cus, hipStream_t s, bool* supported) {
#define TQ_DEC_CASE(BB) \
    case BB: return bf ? launch_one_qjl<D, BB, true>(a, num_cus, s, supported) : launch_one_qjl<D, BB, false>(a, num_cus, s, supported);
    switch (a.t.b) {
        TQ_DEC_CASE(1) TQ_DEC_CASE(2) TQ_DEC_CASE(3) TQ_DEC_CASE(4)
        TQ_DEC_CASE(5) TQ_DEC_CASE(6) TQ_DEC_CASE(7) TQ_DEC_CASE(8)
    }
#undef TQ_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_qjl(const DecodeArgs& a, bool out_bf16, int num_cus, hipStream_t s, bool* supported) {
    switch (a.t.d) {
        case 64: return launch_d_qjl<64>(a, out_bf16, num_cus, s, supported);
        case 128: return launch_d_qjl<128>(a, out_bf16, num_cus, s, supported);
        case 256: return launch_d_qjl<256>(a, out_bf16, num_cus, s, supported);
    }
    return hipErrorInvalidValue;
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
