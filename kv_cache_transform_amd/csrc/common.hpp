// Device building blocks shared by the gfx950 kernels.
//
// Vector layout used by the encode/decode kernels ("4 lanes per vector"): lane l of a wave64 works
// on vector v = l % 16 and part g = l / 16.  A vector of d coordinates is split into 4 parts of
// C = d/4 values held in registers ("slots").  The Walsh-Hadamard transform (natural-order Sylvester
// H, "Ablation, Statistical Inference, and Validation for KV-Cache Compression" §2 TurboQuant) is
// separable over the bits of the coordinate index, so it is done as
//   (1) an in-register radix-2 transform over the slot index, then
//   (2) two cross-lane stages that pair part g with g^1 (v_permlane16_swap) and g^2
//       (v_permlane32_swap).  Each swap exchanges one register between lane halves so that the
//       butterfly partners meet in the same lane; the swapped slot bit and the lane bit trade
//       places.
// With input slot s of part g holding coordinate
//   i(s, g) = (s % R) + g·R + (s / R)·(d/4),   R = d/16,
// the output slot s of part g holds coordinate j = g·C + s, i.e. natural order, contiguous per lane.
// Decoding runs the same network on j-ordered input and produces i(s, g)-ordered output.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// the wave's index in its block as a wave-uniform (scalar) value, so that work indices, loop
// bounds and base addresses derived from it stay in SGPRs
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// bf16 pair dot products with an inline zero accumulator (three-operand VOP3P form):
//   dot2_bf16(a, b)        = a.lo*b.lo + a.hi*b.hi
//   dot2_bf16_nhi(a, b)    = a.lo*b.lo - a.hi*b.hi   (neg_hi on the second operand)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float dot2_bf16_nhi(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// (e0 - h.lo, e1 - h.hi) rounded to fp16 and packed, for a packed fp16 pair h and fp32 e0, e1
// (v_fma_mix{lo,hi}_f16: fp32 fma with an fp16 operand, fp16 result into one half)
// (the first instruction leaves the high half of its destination as it was, and the second
// overwrites it, so the destination needs no initial value)
__device__ __forceinline__ uint32_t sub_f16pair_from_f32(uint32_t h, float e0, float e1) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(e0));
    asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(h), "v"(e1));
    return r;
}

// swap rows 1,3 of a with rows 0,2 of b (rows = 16-lane groups)
__device__ __forceinline__ void xswap16(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(f2u(a), f2u(b), false, false);
    a = u2f(r[0]);
    b = u2f(r[1]);
}
// swap lanes 32..63 of a with lanes 0..31 of b
__device__ __forceinline__ void xswap32(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(f2u(a), f2u(b), false, false);
    a = u2f(r[0]);
    b = u2f(r[1]);
}

// in-register radix-2 Hadamard butterflies over slot bits [lo_bit, log2 C)
template <int C, int FIRST_H = 1>
__device__ __forceinline__ void fwht_slots(float (&x)[C]) {
#pragma unroll
    for (int h = FIRST_H; h < C; h <<= 1) {
#pragma unroll
        for (int i = 0; i < C; i += 2 * h) {
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
        }
    }
}

// the same swaps on raw 32-bit words
__device__ __forceinline__ void xswap16u(uint32_t& a, uint32_t& b) {
    auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void xswap32u(uint32_t& a, uint32_t& b) {
    auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// the two cross-lane stages (see the header comment)
template <int C>
__device__ __forceinline__ void fwht_cross(float (&x)[C]) {
    constexpr int hA = C / 4, hB = C / 2;
#pragma unroll
    for (int s = 0; s < C; ++s) {
        if (s & hA) continue;
        xswap16(x[s], x[s + hA]);
        const float a = x[s], b = x[s + hA];
        x[s] = a + b;
        x[s + hA] = a - b;
    }
#pragma unroll
    for (int s = 0; s < C; ++s) {
        if (s & hB) continue;
        xswap32(x[s], x[s + hB]);
        const float a = x[s], b = x[s + hB];
        x[s] = a + b;
        x[s + hB] = a - b;
    }
}

// sum over the 4 parts of a vector (lanes v, v+16, v+32, v+48); every part gets the total
__device__ __forceinline__ float sum4(float t) {
    float a = t, b = t;
    xswap16(a, b);
    t = a + b;
    a = t;
    b = t;
    xswap32(a, b);
    return a + b;
}

// coordinate index of input slot s in part g (the encode input / decode output order)
__host__ __device__ constexpr int in_coord(int d, int s, int g) {
    return (s % (d / 16)) + g * (d / 16) + (s / (d / 16)) * (d / 4);
}

// ---- bit fields in a little-endian word array ---------------------------------------------------
// `pos` must fold to a constant after unrolling so the word index stays in registers.
template <int NB, int NW>
__device__ __forceinline__ uint32_t get_bits(const uint32_t (&w)[NW], int pos) {
    const int wi = pos >> 5, sh = pos & 31;
    constexpr uint32_t mask = NB >= 32 ? 0xffffffffu : ((1u << NB) - 1u);
    if (sh + NB <= 32) {
        if (sh == 0 && NB == 32) return w[wi];
        return __builtin_amdgcn_ubfe(w[wi], sh, NB);
    }
    return __builtin_amdgcn_alignbit(w[wi + 1 < NW ? wi + 1 : wi], w[wi], sh) & mask;
}

template <int NB, int NW>
__device__ __forceinline__ void put_bits(uint32_t (&w)[NW], int pos, uint32_t v) {
    const int wi = pos >> 5, sh = pos & 31;
    w[wi] |= v << sh;
    if (sh + NB > 32 && wi + 1 < NW) w[wi + 1] |= v >> (32 - sh);
}

// ---- vector memory helpers: NB bytes, alignment A (bytes, power of two <= 16) -----------------
template <int NB, int A>
__device__ __forceinline__ void store_bytes(uint8_t* p, const uint32_t* w) {
    if constexpr (A == 1) {
#pragma unroll
        for (int i = 0; i < NB; ++i) p[i] = (uint8_t)(w[i / 4] >> (8 * (i % 4)));
    } else if constexpr (A >= 16 && NB >= 16) {
        *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
        if constexpr (NB > 16) store_bytes<NB - 16, 16>(p + 16, w + 4);
    } else if constexpr (A >= 8 && NB >= 8) {
        *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
        if constexpr (NB > 8) store_bytes<NB - 8, (A > 8 ? 8 : A)>(p + 8, w + 2);
    } else if constexpr (A >= 4 && NB >= 4) {
        *reinterpret_cast<uint32_t*>(p) = w[0];
        if constexpr (NB > 4) store_bytes<NB - 4, 4>(p + 4, w + 1);
    } else if constexpr (NB >= 2) {
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)(w[0] & 0xffffu);
        if constexpr (NB >= 4) *reinterpret_cast<uint16_t*>(p + 2) = (uint16_t)(w[0] >> 16);
        if constexpr (NB > 4) store_bytes<NB - 4, 2>(p + 4, w + 1);
        else if constexpr (NB == 3) p[2] = (uint8_t)(w[0] >> 16);
    } else if constexpr (NB == 1) {
        p[0] = (uint8_t)(w[0] & 0xffu);
    }
}

template <int NB, int A>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* w) {
    if constexpr (A == 1) {
#pragma unroll
        for (int i = 0; i < (NB + 3) / 4; ++i) w[i] = 0u;
#pragma unroll
        for (int i = 0; i < NB; ++i) w[i / 4] |= uint32_t(p[i]) << (8 * (i % 4));
    } else if constexpr (A >= 16 && NB >= 16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
        if constexpr (NB > 16) load_bytes<NB - 16, 16>(p + 16, w + 4);
    } else if constexpr (A >= 8 && NB >= 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        w[0] = v[0]; w[1] = v[1];
        if constexpr (NB > 8) load_bytes<NB - 8, (A > 8 ? 8 : A)>(p + 8, w + 2);
    } else if constexpr (A >= 4 && NB >= 4) {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
        if constexpr (NB > 4) load_bytes<NB - 4, 4>(p + 4, w + 1);
    } else if constexpr (NB >= 2) {
        uint32_t lo = *reinterpret_cast<const uint16_t*>(p);
        if constexpr (NB >= 4) lo |= uint32_t(*reinterpret_cast<const uint16_t*>(p + 2)) << 16;
        else if constexpr (NB == 3) lo |= uint32_t(p[2]) << 16;
        w[0] = lo;
        if constexpr (NB > 4) load_bytes<NB - 4, 2>(p + 4, w + 1);
    } else if constexpr (NB == 1) {
        w[0] = p[0];
    }
}

// ---- raw buffer access: a resource over one byte range, 32-bit per-lane and wave-uniform offsets --
// A raw buffer (stride 0) over [base, base + bytes): the address is the base plus the offsets, with no
// per-lane 64-bit arithmetic, and an access whose per-lane offset reaches `bytes` reads 0 or is not
// written.  bytes = 0xffffffff (as int, -1) leaves the range unchecked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes = -1) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// NB bytes at byte offset voff (per lane) + soff (wave-uniform) of buffer r, alignment A (a
// power of two <= 16): raw buffer loads, so the address is the resource base plus two 32-bit
// offsets and needs no per-lane 64-bit arithmetic
template <int NB, int A>
__device__ __forceinline__ void bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w) {
    if constexpr (A >= 16 && NB >= 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
        if constexpr (NB > 16) bload<NB - 16, 16>(r, voff + 16, soff, w + 4);
    } else if constexpr (A >= 8 && NB >= 8) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        w[0] = v[0]; w[1] = v[1];
        if constexpr (NB > 8) bload<NB - 8, (A > 8 ? 8 : A)>(r, voff + 8, soff, w + 2);
    } else if constexpr (A >= 4 && NB >= 4) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        if constexpr (NB > 4) bload<NB - 4, 4>(r, voff + 4, soff, w + 1);
    } else if constexpr (NB >= 2) {
        uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
        if constexpr (NB >= 4) lo |= uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, voff + 2, soff, 0)) << 16;
        else if constexpr (NB == 3) lo |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(r, voff + 2, soff, 0)) << 16;
        w[0] = lo;
        if constexpr (NB > 4) bload<NB - 4, 2>(r, voff + 4, soff, w + 1);
    } else if constexpr (NB == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
    }
}

// NB bytes from w to byte offset voff (per lane) + soff (wave-uniform) of buffer r, alignment A
template <int NB, int A>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const uint32_t* w) {
    if constexpr (A >= 16 && NB >= 16) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, r, voff, soff, 0);
        if constexpr (NB > 16) bstore<NB - 16, 16>(r, voff + 16, soff, w + 4);
    } else if constexpr (A >= 8 && NB >= 8) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, r, voff, soff, 0);
        if constexpr (NB > 8) bstore<NB - 8, (A > 8 ? 8 : A)>(r, voff + 8, soff, w + 2);
    } else if constexpr (A >= 4 && NB >= 4) {
        __builtin_amdgcn_raw_buffer_store_b32(w[0], r, voff, soff, 0);
        if constexpr (NB > 4) bstore<NB - 4, 4>(r, voff + 4, soff, w + 1);
    } else if constexpr (NB >= 2) {
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[0] & 0xffffu), r, voff, soff, 0);
        if constexpr (NB >= 4) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[0] >> 16), r, voff + 2, soff, 0);
        else if constexpr (NB == 3) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w[0] >> 16), r, voff + 2, soff, 0);
        if constexpr (NB > 4) bstore<NB - 4, 2>(r, voff + 4, soff, w + 1);
    } else if constexpr (NB == 1) {
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w[0] & 0xffu), r, voff, soff, 0);
    }
}

constexpr int pow2_align(int x) { return (x % 16 == 0) ? 16 : (x % 8 == 0) ? 8 : (x % 4 == 0) ? 4 : (x % 2 == 0) ? 2 : 1; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// coordinates per dequantisation lookup for b bits (matches the host LUT builder)
constexpr int lut_group_c(int b) { return (b == 1 || b == 2 || b == 4) ? 8 / b : ((b == 3 || b == 5 || b == 6) ? 2 : 1); }

}  // namespace tq
