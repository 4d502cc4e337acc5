// Fourier-magnitude codec, host side: the DFT and inverse-DFT operand tiles, the phase-level
// table, the query-side tables of the scores, and the C ABI of include/tq_fmag.h ("Fourier Magnitude
// KV Cache Quantization", forum thread, "Method").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "../../include/tq_fmag.h"
#include "fmag_kernels.hpp"
#include "tables.hpp"

namespace tq {
namespace {

int check(const tq_fmag_params* p) {
    if (!p) return TQ_EINVAL;
    if (p->d != 64 && p->d != 128) return TQ_EINVAL;
    if (p->b < 1 || p->b > 8) return TQ_EINVAL;
    if (!((p->p >= 1 && p->p <= 8) || p->p == TQ_FMAG_PHASE_BF16)) return TQ_EINVAL;
    return TQ_OK;
}

int record_words(const tq_fmag_params* p) {
    const int nb = p->d / 2 + 1;
    return (nb * (p->b + p->p) + 31) / 32 + 2;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// DFT coefficient of input j for spectrum coordinate c (X_c = Σ_j F(j, c) x_j) and the inverse
// coefficient (x_j = Σ_c G(j, c) X_c) in the coordinate order of fmag_kernels.hpp
double dft_coef(int d, int j, int c) {
    if (c < d / 2) return std::cos(2.0 * M_PI * j * c / d);
    if (c == d / 2) return (j & 1) ? -1.0 : 1.0;
    return -std::sin(2.0 * M_PI * j * (c - d / 2) / d);
}
double idft_coef(int d, int j, int c) {
    if (c == 0) return 1.0 / d;
    if (c < d / 2) return 2.0 / d * std::cos(2.0 * M_PI * j * c / d);
    if (c == d / 2) return ((j & 1) ? -1.0 : 1.0) / d;
    return -2.0 / d * std::sin(2.0 * M_PI * j * (c - d / 2) / d);
}

void split16(double v, uint16_t* hi, uint16_t* lo) {
    *hi = f64_to_f16_bits(v);
    *lo = f64_to_f16_bits(v - (double)f16_bits_to_f32(*hi));
}

using Key = std::tuple<int, int, int, int>;   // device, d, b, p
std::mutex g_mu;
std::map<Key, FmDev> g_tables;
std::map<int, int> g_cus;

int build(const tq_fmag_params* p, FmDev* out) {
    const int d = p->d, T = d / 16, S = d / 32;
    std::vector<uint16_t> enc((size_t)2 * T * S * 512), dec((size_t)2 * T * S * 512);
    const double gmax = 2.0 / d;
    const int e = 13 - (int)std::floor(std::log2(gmax));
    for (int t = 0; t < T; ++t)
        for (int s = 0; s < S; ++s)
            for (int l = 0; l < 64; ++l)
                for (int i = 0; i < 8; ++i) {
                    const size_t o = (((size_t)t * S + s) * 64 + l) * 8 + i, lo_off = (size_t)T * S * 512;
                    // encode B[kk = 8g + i][n = l % 16]: input j = 32 s + 8 g + i, coordinate c = 16 t + n
                    split16(dft_coef(d, 32 * s + 8 * (l / 16) + i, 16 * t + (l % 16)) * 256.0, &enc[o], &enc[o + lo_off]);
                    // decode A[m = l % 16][kk = 8 g + i]: output j = 16 t + m, coordinate c = 32 s + 8 g + i
                    split16(std::ldexp(idft_coef(d, 16 * t + (l % 16), 32 * s + 8 * (l / 16) + i), e), &dec[o],
                            &dec[o + lo_off]);
                }
    std::vector<float> cs(512, 0.0f);
    if (p->p <= 8)
        for (int i = 0; i < (1 << p->p); ++i) {
            const double a = -M_PI + 2.0 * M_PI * i / (1 << p->p);
            cs[2 * i] = (float)std::cos(a);
            cs[2 * i + 1] = (float)std::sin(a);
        }
    std::vector<float> U((size_t)d * d), w(d), G((size_t)d * d);
    for (int j = 0; j < d; ++j)
        for (int c = 0; c < d; ++c) {
            U[(size_t)j * d + c] = (float)dft_coef(d, j, c);
            G[(size_t)j * d + c] = (float)idft_coef(d, j, c);
        }
    for (int c = 0; c < d; ++c) w[c] = (float)((c == 0 || c == d / 2 ? 1.0 : 2.0) / d);

    size_t off = 0;
    auto place = [&](size_t bytes) { const size_t o = off; off = (off + bytes + 255) / 256 * 256; return o; };
    const size_t o_e = place(enc.size() * 2), o_d = place(dec.size() * 2), o_c = place(cs.size() * 4),
                 o_u = place(U.size() * 4), o_w = place(w.size() * 4), o_g = place(G.size() * 4);
    std::vector<uint8_t> blob(off);
    std::memcpy(blob.data() + o_e, enc.data(), enc.size() * 2);
    std::memcpy(blob.data() + o_d, dec.data(), dec.size() * 2);
    std::memcpy(blob.data() + o_c, cs.data(), cs.size() * 4);
    std::memcpy(blob.data() + o_u, U.data(), U.size() * 4);
    std::memcpy(blob.data() + o_w, w.data(), w.size() * 4);
    std::memcpy(blob.data() + o_g, G.data(), G.size() * 4);
    void* mem = nullptr;
    if (hipMalloc(&mem, blob.size()) != hipSuccess) return TQ_EHIP;
    if (hipMemcpy(mem, blob.data(), blob.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(mem);
        return TQ_EHIP;
    }
    uint8_t* base = static_cast<uint8_t*>(mem);
    FmDev t;
    t.d = d;
    t.b = p->b;
    t.p = p->p;
    t.rec_words = record_words(p);
    t.enc_b = reinterpret_cast<const _Float16*>(base + o_e);
    t.dec_a = reinterpret_cast<const _Float16*>(base + o_d);
    t.dec_scale = (float)std::ldexp(1.0, -e);
    t.cs = reinterpret_cast<const float*>(base + o_c);
    t.qprep.d = d;
    t.qprep.n_heads = 1;
    t.qprep.U32 = reinterpret_cast<const float*>(base + o_u);
    t.qprep.sigma = reinterpret_cast<const float*>(base + o_w);
    t.G32 = reinterpret_cast<const float*>(base + o_g);
    t.blob = mem;
    *out = t;
    return TQ_OK;
}

int tables(const tq_fmag_params* p, FmDev* out, int* cus) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return TQ_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto c = g_cus.find(device);
    if (c == g_cus.end()) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return TQ_EHIP;
        c = g_cus.emplace(device, n).first;
    }
    *cus = c->second;
    const Key key{device, p->d, p->b, p->p};
    auto it = g_tables.find(key);
    if (it == g_tables.end()) {
        FmDev t;
        const int rc = build(p, &t);
        if (rc != TQ_OK) return rc;
        it = g_tables.emplace(key, t).first;
    }
    *out = it->second;
    return TQ_OK;
}

// attention split geometry, a function of the arguments only: about as many (stream, split) waves
// as 256 CUs hold (twelve per CU, three per SIMD; eight when a record exceeds 28 words, whose
// kernel runs at two per SIMD), splits of at least 256 tokens in multiples of 32, at most 1024
struct AttnWs {
    int64_t tps, n_split, o_qlo, o_qs, o_part, o_ml, total;
};
int64_t waves_per_cu(const tq_fmag_params* pk, const tq_fmag_params* pv) {
    return (pk->d == 64 || std::max(record_words(pk), record_words(pv)) <= 28) ? 12 : 8;
}
AttnWs attn_ws(int d, int64_t per_cu, int64_t streams, int64_t n_tokens) {
    AttnWs w{};
    int64_t ns = (256 * per_cu + streams - 1) / (streams > 0 ? streams : 1);
    ns = std::min(ns, (n_tokens + 255) / 256);
    ns = std::max<int64_t>(std::min<int64_t>(ns, 1024), 1);
    w.tps = std::max<int64_t>(((n_tokens + ns - 1) / ns + 31) / 32 * 32, 32);
    w.n_split = std::max<int64_t>((n_tokens + w.tps - 1) / w.tps, 1);
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    w.o_qlo = al(streams * 16 * d * 2);
    w.o_qs = w.o_qlo + al(streams * 16 * d * 2);
    w.o_part = w.o_qs + al(streams * 16 * 4);
    w.o_ml = w.o_part + al(streams * w.n_split * 16 * d * 4);
    w.total = w.o_ml + al(streams * w.n_split * 16 * 2 * 4);
    return w;
}

}  // namespace

// frees the Fmag tables (called by tq_clear_cache)
void fmag_clear_tables() {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_tables) (void)hipFree(kv.second.blob);
    g_tables.clear();
}

}  // namespace tq

using namespace tq;

extern "C" {

int tq_fmag_record_bytes(const tq_fmag_params* p, int64_t* bytes) {
    if (check(p) != TQ_OK || !bytes) return TQ_EINVAL;
    *bytes = (int64_t)record_words(p) * 4;
    return TQ_OK;
}

int tq_fmag_encode(const tq_fmag_params* p, const void* x, tq_dtype x_dtype, int64_t n_streams,
                   int64_t n_tokens, void* packed, void* stream) {
    if (check(p) != TQ_OK || n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    if (x_dtype != TQ_BF16) return x_dtype == TQ_F32 || x_dtype == TQ_F16 ? TQ_EUNSUPPORTED : TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0) return TQ_OK;
    if (!x || !packed) return TQ_EINVAL;
    if (!aligned16(x) || !aligned16(packed)) return TQ_EALIGN;
    FmEncodeArgs a{};
    int cus = 0;
    const int rc = tables(p, &a.t, &cus);
    if (rc != TQ_OK) return rc;
    a.x = static_cast<const uint16_t*>(x);
    a.out = static_cast<uint32_t*>(packed);
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    return launch_fmag_encode(a, cus, static_cast<hipStream_t>(stream)) == hipSuccess ? TQ_OK : TQ_EHIP;
}

int tq_fmag_decode(const tq_fmag_params* p, const void* packed, int64_t n_streams, int64_t n_tokens,
                   void* x_hat, tq_dtype out_dtype, void* stream) {
    if (check(p) != TQ_OK || n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return out_dtype == TQ_F16 ? TQ_EUNSUPPORTED : TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0) return TQ_OK;
    if (!packed || !x_hat) return TQ_EINVAL;
    if (!aligned16(packed) || !aligned16(x_hat)) return TQ_EALIGN;
    FmDecodeArgs a{};
    int cus = 0;
    const int rc = tables(p, &a.t, &cus);
    if (rc != TQ_OK) return rc;
    a.in = static_cast<const uint32_t*>(packed);
    a.out = x_hat;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    return launch_fmag_decode(a, out_dtype == TQ_BF16, cus, static_cast<hipStream_t>(stream)) == hipSuccess ? TQ_OK
                                                                                                            : TQ_EHIP;
}

size_t tq_fmag_scores_workspace_bytes(const tq_fmag_params* p, int64_t n_streams, int64_t n_q) {
    if (check(p) != TQ_OK || n_streams < 0 || n_q < 0) return 0;
    const int64_t nq_pad = (n_q + 15) / 16 * 16;
    const int64_t qp = (n_streams * nq_pad * p->d * 2 + 255) / 256 * 256;
    return (size_t)(2 * qp + (n_streams * nq_pad * 4 + 255) / 256 * 256);
}

int tq_fmag_qk_scores(const tq_fmag_params* p, const void* q, tq_dtype q_dtype, int64_t n_q,
                      const void* packed, int64_t n_streams, int64_t n_tokens, float* scores,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (check(p) != TQ_OK || n_streams < 0 || n_tokens < 0 || n_q < 0 || n_q > 256) return TQ_EINVAL;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return q_dtype == TQ_F16 ? TQ_EUNSUPPORTED : TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0 || n_q == 0) return TQ_OK;
    if (!q || !packed || !scores || !workspace) return TQ_EINVAL;
    if (!aligned16(q) || !aligned16(packed) || !aligned16(scores) || !aligned16(workspace)) return TQ_EALIGN;
    if (workspace_bytes < tq_fmag_scores_workspace_bytes(p, n_streams, n_q)) return TQ_EWORKSPACE;
    FmScoresArgs a{};
    int cus = 0;
    const int rc = tables(p, &a.t, &cus);
    if (rc != TQ_OK) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nq_pad = (n_q + 15) / 16 * 16;
    const int64_t qpb = (n_streams * nq_pad * p->d * 2 + 255) / 256 * 256;
    SqScoresArgs qa{};
    qa.t = a.t.qprep;
    qa.q = q;
    qa.q_bf16 = q_dtype == TQ_BF16;
    qa.qp = static_cast<_Float16*>(workspace);
    qa.qplo = reinterpret_cast<_Float16*>(static_cast<uint8_t*>(workspace) + qpb);
    qa.qscale = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + 2 * qpb);
    qa.qmul = 1.0f;
    qa.n_streams = n_streams;
    qa.n_q = n_q;
    qa.nq_pad = nq_pad;
    if (launch_sq_qprep(qa, s) != hipSuccess) return TQ_EHIP;
    a.qp = qa.qp;
    a.qplo = qa.qplo;
    a.qscale = qa.qscale;
    a.in = static_cast<const uint32_t*>(packed);
    a.scores = scores;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.n_q = n_q;
    a.nq_pad = nq_pad;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    return launch_fmag_scores(a, cus, s) == hipSuccess ? TQ_OK : TQ_EHIP;
}

size_t tq_fmag_attention_workspace_bytes(const tq_fmag_params* pk, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t n_tokens) {
    if (check(pk) != TQ_OK || batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_tokens < 0) return 0;
    // sized for the larger geometry (the value codec may allow it): an upper bound for any V
    return (size_t)attn_ws(pk->d, 12, (int64_t)batch * n_kv_heads, n_tokens).total;
}

int tq_fmag_decode_attention(const tq_fmag_params* pk, const tq_fmag_params* pv, const void* q, tq_dtype q_dtype,
                             int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                             const void* packed_v, int64_t n_tokens, const int32_t* lengths, float softmax_scale,
                             void* out, tq_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (check(pk) != TQ_OK || check(pv) != TQ_OK || pk->d != pv->d) return TQ_EINVAL;
    if (batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_tokens < 0) return TQ_EINVAL;
    if (n_q_heads % n_kv_heads != 0 || n_q_heads / n_kv_heads > 16) return TQ_EINVAL;
    if ((q_dtype != TQ_F32 && q_dtype != TQ_BF16) || (out_dtype != TQ_F32 && out_dtype != TQ_BF16)) {
        const bool known = q_dtype == TQ_F16 || out_dtype == TQ_F16;
        return known ? TQ_EUNSUPPORTED : TQ_EINVAL;
    }
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f) return TQ_EINVAL;
    if (batch == 0) return TQ_OK;
    if (!q || !out || !workspace || (n_tokens > 0 && (!packed_k || !packed_v))) return TQ_EINVAL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(workspace) ||
        (n_tokens > 0 && (!aligned16(packed_k) || !aligned16(packed_v))))
        return TQ_EALIGN;
    if (lengths && (reinterpret_cast<uintptr_t>(lengths) & 3u)) return TQ_EALIGN;
    const int64_t streams = (int64_t)batch * n_kv_heads;
    const AttnWs w = attn_ws(pk->d, waves_per_cu(pk, pv), streams, n_tokens);
    if (workspace_bytes < (size_t)w.total) return TQ_EWORKSPACE;
    FmAttnArgs a{};
    int cus = 0;
    int rc = tables(pk, &a.tk, &cus);
    if (rc != TQ_OK) return rc;
    rc = tables(pv, &a.tv, &cus);
    if (rc != TQ_OK) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)pk->d);
    SqScoresArgs qa{};
    qa.t = a.tk.qprep;
    qa.q = q;
    qa.q_bf16 = q_dtype == TQ_BF16;
    qa.qp = reinterpret_cast<_Float16*>(ws);
    qa.qplo = reinterpret_cast<_Float16*>(ws + w.o_qlo);
    qa.qscale = reinterpret_cast<float*>(ws + w.o_qs);
    qa.qmul = scale * 1.4426950408889634f;   // scores in base-2 units for exp2
    qa.n_streams = streams;
    qa.n_q = n_q_heads / n_kv_heads;
    qa.nq_pad = 16;
    if (launch_sq_qprep(qa, s) != hipSuccess) return TQ_EHIP;
    a.qp = qa.qp;
    a.qplo = qa.qplo;
    a.qscale = qa.qscale;
    a.kin = static_cast<const uint32_t*>(packed_k);
    a.vin = static_cast<const uint32_t*>(packed_v);
    a.lens = lengths;
    a.part = reinterpret_cast<float*>(ws + w.o_part);
    a.ml = reinterpret_cast<float*>(ws + w.o_ml);
    a.out = out;
    a.out_bf16 = out_dtype == TQ_BF16;
    a.n_streams = streams;
    a.n_tokens = n_tokens;
    a.tps = w.tps;
    a.n_split = w.n_split;
    a.hkv = n_kv_heads;
    a.hq = n_q_heads;
    a.g = n_q_heads / n_kv_heads;
    return launch_fmag_attention(a, s) == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // extern "C"
