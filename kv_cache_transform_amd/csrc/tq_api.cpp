// C ABI of libtq (declared in include/tq.h): argument validation, packed layout, the device table
// cache and kernel dispatch.  Every entry point validates all arguments before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <tuple>
#include <vector>

#include "../../include/tq.h"
#include "fmag_kernels.hpp"
#include "kernels.hpp"
#include "tables.hpp"

namespace tq {
namespace {

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_params(const tq_params* p) {
    if (!p) return TQ_EINVAL;
    if (p->d != 64 && p->d != 128 && p->d != 256) return TQ_EINVAL;
    if (p->b < 1 || p->b > 8) return TQ_EINVAL;
    if (p->m < 0 || p->m % 32 != 0 || p->m > p->d) return TQ_EINVAL;
    if (p->n_heads < 1) return TQ_EINVAL;
    if (p->sketch != TQ_SKETCH_GAUSSIAN && p->sketch != TQ_SKETCH_RHT) return TQ_EINVAL;
    if (p->sketch == TQ_SKETCH_RHT && p->m != 0 && p->m != p->d) return TQ_EINVAL;
    if (p->rotation != TQ_ROTATION_WHT && p->rotation != TQ_ROTATION_NONE) return TQ_EINVAL;
    return TQ_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

void layout_of(const tq_params* p, int64_t n_streams, int64_t n_tokens, tq_layout* o) {
    const int64_t nv = n_streams * n_tokens;
    o->idx_bytes_per_vec = (int64_t)p->d * p->b / 8;
    o->sketch_bytes_per_vec = p->m / 8;
    o->off_idx = 0;
    o->off_sketch = align_up(o->off_idx + nv * o->idx_bytes_per_vec);
    o->off_norm = align_up(o->off_sketch + nv * o->sketch_bytes_per_vec);
    o->off_rnorm = align_up(o->off_norm + nv * 2);
    o->total_bytes = align_up(o->off_rnorm + (p->m > 0 ? nv * 2 : 0));
}

// ---- host codebook cache (per d, b) -----------------------------------------------------------
struct Codebook {
    std::vector<double> thr, cent;
};
std::mutex g_mu;
std::map<std::pair<int, int>, Codebook> g_codebooks;

const Codebook& codebook(int d, int b) {  // caller holds g_mu
    auto key = std::make_pair(d, b);
    auto it = g_codebooks.find(key);
    if (it != g_codebooks.end()) return it->second;
    Codebook cb;
    lloyd_max(d, b, cb.thr, cb.cent);
    return g_codebooks.emplace(key, std::move(cb)).first->second;
}

// ---- device table cache ----------------------------------------------------------------------
using TableKey = std::tuple<int, int, int, int, int, uint64_t, int, int>;  // device, d, b, m, n_heads, seed, sketch, rotation
std::map<TableKey, DevTables> g_tables;
std::map<int, int> g_num_cus;

struct Blob {
    std::vector<uint8_t> host;
    int64_t add(const void* src, int64_t bytes) {
        const int64_t off = align_up((int64_t)host.size());
        host.resize(off + align_up(bytes));
        std::memcpy(host.data() + off, src, bytes);
        return off;
    }
};

int build_tables(const tq_params* p, int device, DevTables* out) {  // caller holds g_mu
    const int d = p->d, b = p->b, m = p->m, H = p->n_heads, L = 1 << b, C = d / 4;
    const Codebook& cb = codebook(d, b);
    std::vector<float> cent_f(L), cent_k(L);
    for (int i = 0; i < L; ++i) {
        cent_f[i] = (float)cb.cent[i];
        cent_k[i] = cent_f[i] * 16384.0f;
    }
    Grid grid;
    if (!build_grid(cb.thr, grid)) return TQ_EUNSUPPORTED;
    const std::vector<uint32_t>& gw = grid.entries;
    std::vector<uint32_t> fq;
    const bool fq_ok = build_fq_grid(cb.thr, b, fq);

    const int P = lut_group(b), NE = 1 << (P * b);
    std::vector<float> lut32((size_t)NE * P);
    std::vector<uint16_t> lut16((size_t)NE * P), luthl((size_t)NE * P * 2);
    for (int f = 0; f < NE; ++f)
        for (int k = 0; k < P; ++k) {
            const int idx = (f >> (k * b)) & (L - 1);
            lut32[(size_t)f * P + k] = cent_f[idx];
            lut16[(size_t)f * P + k] = f32_to_f16_bits(cent_f[idx]);
            // fp16 hi + lo of 2^12 c, = 2^12 times the fp32 centroid to 2^-22 relative (the difference
            // is exact; the 2^12 keeps lo out of the fp16 subnormal range)
            const float cs = cent_f[idx] * 4096.0f;
            const uint16_t hi = f32_to_f16_bits(cs);
            luthl[(size_t)f * 2 * P + k] = hi;
            luthl[(size_t)f * 2 * P + P + k] = f32_to_f16_bits(cs - f16_bits_to_f32(hi));
        }

    const bool rht = m > 0 && p->sketch == TQ_SKETCH_RHT;
    std::vector<float> signs((size_t)H * d), signs_slot((size_t)H * d), signs2(rht ? (size_t)H * d : 0), sh;
    std::vector<uint16_t> S((size_t)H * m * d), Sh;
    for (int h = 0; h < H; ++h) {
        head_signs(p->seed, h, d, sh);
        std::memcpy(&signs[(size_t)h * d], sh.data(), d * 4);
        for (int g = 0; g < 4; ++g)
            for (int s = 0; s < C; ++s) {
                const int i = (s % (d / 16)) + g * (d / 16) + (s / (d / 16)) * (d / 4);
                signs_slot[((size_t)h * 4 + g) * C + s] = sh[i];
            }
        if (m > 0) {
            if (rht) {
                rht_matrix_f16(p->seed, h, d, Sh);
                rht_signs(p->seed, h, d, sh);
                std::memcpy(&signs2[(size_t)h * d], sh.data(), d * 4);
            } else {
                gaussian_matrix_f16(p->seed, h, m, d, Sh);
            }
            std::memcpy(&S[(size_t)h * m * d], Sh.data(), (size_t)m * d * 2);
        }
    }

    Blob blob;
    const int64_t o_grid = blob.add(gw.data(), gw.size() * 4);
    const int64_t o_fq = fq_ok ? blob.add(fq.data(), fq.size() * 4) : 0;
    const int64_t o_cent = blob.add(cent_f.data(), L * 4);
    const int64_t o_centk = blob.add(cent_k.data(), L * 4);
    const int64_t o_l32 = blob.add(lut32.data(), lut32.size() * 4);
    const int64_t o_l16 = blob.add(lut16.data(), lut16.size() * 2);
    const int64_t o_lhl = blob.add(luthl.data(), luthl.size() * 2);
    const int64_t o_ss = blob.add(signs_slot.data(), signs_slot.size() * 4);
    const int64_t o_sg = blob.add(signs.data(), signs.size() * 4);
    const int64_t o_S = m > 0 ? blob.add(S.data(), S.size() * 2) : 0;
    const int64_t o_s2 = rht ? blob.add(signs2.data(), signs2.size() * 4) : 0;
    // the decode-attention's 4-bit table image (see DevTables::attn_img): byte e packs the
    // coordinates (e & 15, e >> 4), P = 2 per LUT entry, so the key pairs are lut_hl's words 2e, 2e + 1
    std::vector<uint32_t> img(b == 4 ? (size_t)2 * 256 * 64 : 0);
    if (b == 4) {
        for (int e = 0; e < 256; ++e) {
            const uint32_t vp = (uint32_t)lut16[(size_t)e * 2] | ((uint32_t)lut16[(size_t)e * 2 + 1] << 16);
            const uint32_t kh = (uint32_t)luthl[(size_t)e * 4] | ((uint32_t)luthl[(size_t)e * 4 + 1] << 16);
            const uint32_t kl = (uint32_t)luthl[(size_t)e * 4 + 2] | ((uint32_t)luthl[(size_t)e * 4 + 3] << 16);
            for (int c = 0; c < 32; ++c) {
                img[(size_t)e * 64 + c] = vp;
                img[(size_t)e * 64 + 32 + c] = kh;
                img[(size_t)(256 + e) * 64 + c] = kl;
                img[(size_t)(256 + e) * 64 + 32 + c] = 0u;
            }
        }
    }
    const int64_t o_img = b == 4 ? blob.add(img.data(), img.size() * 4) : 0;

    void* dev = nullptr;
    if (hipMalloc(&dev, blob.host.size()) != hipSuccess) return TQ_EHIP;
    if (hipMemcpy(dev, blob.host.data(), blob.host.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dev);
        return TQ_EHIP;
    }
    uint8_t* base = static_cast<uint8_t*>(dev);
    DevTables t;
    t.d = d; t.b = b; t.m = m; t.n_heads = H; t.seed = p->seed; t.sketch = rht ? TQ_SKETCH_RHT : TQ_SKETCH_GAUSSIAN; t.rotation = p->rotation;
    t.G = grid.G;
    t.grid = reinterpret_cast<const uint32_t*>(base + o_grid);
    t.fq_grid = fq_ok ? reinterpret_cast<const uint32_t*>(base + o_fq) : nullptr;
    t.cent = reinterpret_cast<const float*>(base + o_cent);
    t.cent_x1024 = reinterpret_cast<const float*>(base + o_centk);
    t.lut_f32 = reinterpret_cast<const float*>(base + o_l32);
    t.lut_f16 = reinterpret_cast<const _Float16*>(base + o_l16);
    t.lut_hl = reinterpret_cast<const _Float16*>(base + o_lhl);
    t.signs_slot = reinterpret_cast<const float*>(base + o_ss);
    t.signs = reinterpret_cast<const float*>(base + o_sg);
    t.S = m > 0 ? reinterpret_cast<const _Float16*>(base + o_S) : nullptr;
    t.signs2 = rht ? reinterpret_cast<const float*>(base + o_s2) : nullptr;
    t.attn_img = b == 4 ? reinterpret_cast<const uint32_t*>(base + o_img) : nullptr;
    t.blob = dev;
    (void)device;
    *out = t;
    return TQ_OK;
}

// CU count of the current device (cached)
int device_cus(int* cus) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return TQ_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto nc = g_num_cus.find(device);
    if (nc == g_num_cus.end()) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return TQ_EHIP;
        nc = g_num_cus.emplace(device, n).first;
    }
    *cus = nc->second;
    return TQ_OK;
}

// the resident tables of `p` on the current device, without building them (TQ_EUNSUPPORTED if a
// call with these parameters has not built them yet on this device): no allocation on this path
int find_tables(const tq_params* p, DevTables* out, int* num_cus) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return TQ_EHIP;
    if (device_cus(num_cus) != TQ_OK) return TQ_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_tables.find(TableKey{device, p->d, p->b, p->m, p->n_heads, p->seed, p->sketch, p->rotation});
    if (it == g_tables.end()) return TQ_EUNSUPPORTED;
    *out = it->second;
    return TQ_OK;
}

int get_tables(const tq_params* p, DevTables* out, int* num_cus) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return TQ_EHIP;
    if (device_cus(num_cus) != TQ_OK) return TQ_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    const TableKey key{device, p->d, p->b, p->m, p->n_heads, p->seed, p->sketch, p->rotation};
    auto it = g_tables.find(key);
    if (it != g_tables.end()) {
        *out = it->second;
        return TQ_OK;
    }
    DevTables t;
    const int rc = build_tables(p, device, &t);
    if (rc != TQ_OK) return rc;
    g_tables.emplace(key, t);
    *out = t;
    return TQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EHIP; }

// attention split geometry (shared by the workspace query and the launch, and a function of the
// arguments only so the workspace size needs no device): one wave per (stream, split), as many
// waves as a 256-CU MI355X holds at once (two 4-wave blocks per CU for d <= 128, one for d = 256),
// so every wave streams one long token range; at least 256 tokens per split, token ranges a
// multiple of 32, at most 1024 splits
constexpr int kAttnCUs = 256;
// waves per CU of the attention kernel: 12 for 4-bit keys and values at d <= 128 with at most 8
// query heads per kv head (three per SIMD), 8 otherwise at d <= 128, 4 at d = 256
int64_t attn_tokens_per_split(int d, int b, int group, int64_t n_streams, int64_t n_tokens) {
    const int64_t target = (int64_t)kAttnCUs * (d <= 128 ? (b == 4 && group <= 8 ? 12 : 8) : 4);
    int64_t ns = (target + n_streams - 1) / (n_streams > 0 ? n_streams : 1);
    const int64_t max_ns = (n_tokens + 255) / 256;
    if (ns > max_ns) ns = max_ns;
    if (ns > 1024) ns = 1024;
    if (ns < 1) ns = 1;
    int64_t tps = (n_tokens + ns - 1) / ns;
    tps = (tps + 31) / 32 * 32;
    return tps < 32 ? 32 : tps;
}

// query operands of `rows` rows in a workspace starting at byte `base` (see QOps): hi, lo parts of
// the rotated queries and of their sketch projections, then the row factors
struct QOpsLayout {
    int64_t o_qh, o_ql, o_ph, o_pl, o_rf, end;
};
QOpsLayout qops_layout(int64_t base, int64_t rows, int d, int m) {
    QOpsLayout l{};
    const int64_t mm = m > 0 ? m : 1;
    l.o_qh = base;
    l.o_ql = l.o_qh + align_up(rows * d * 2);
    l.o_ph = l.o_ql + align_up(rows * d * 2);
    l.o_pl = l.o_ph + align_up(rows * mm * 2);
    l.o_rf = l.o_pl + align_up(rows * mm * 2);
    l.end = l.o_rf + align_up(rows * 4);
    return l;
}
QOps qops_at(uint8_t* ws, const QOpsLayout& l) {
    QOps o;
    o.qh = reinterpret_cast<_Float16*>(ws + l.o_qh);
    o.ql = reinterpret_cast<_Float16*>(ws + l.o_ql);
    o.ph = reinterpret_cast<_Float16*>(ws + l.o_ph);
    o.pl = reinterpret_cast<_Float16*>(ws + l.o_pl);
    o.rowf = reinterpret_cast<float*>(ws + l.o_rf);
    return o;
}

struct AttnWs {
    QOpsLayout q;
    int64_t o_part, o_ml, total, n_split;
};

AttnWs attn_ws(const tq_params* pk, int32_t batch, int32_t hq, int32_t hkv, int64_t n_tokens) {
    AttnWs w{};
    const int64_t rows = (int64_t)batch * hq + 16;
    const int64_t tps = attn_tokens_per_split(pk->d, pk->b, hkv > 0 ? hq / hkv : 1, (int64_t)batch * hkv, n_tokens);
    w.n_split = (n_tokens + tps - 1) / tps;
    if (w.n_split < 1) w.n_split = 1;
    const int64_t streams = (int64_t)batch * hkv;
    w.q = qops_layout(0, rows, pk->d, pk->m);
    w.o_part = w.q.end;
    w.o_ml = w.o_part + align_up(streams * w.n_split * 16 * pk->d * 4);
    w.total = w.o_ml + align_up(streams * w.n_split * 16 * 2 * 4);
    return w;
}

}  // namespace

// ---- device scratch of the allocation-free attention entry point -------------------------------
// One array per device, for callers that cannot allocate (graph capture, allocation-free serving
// loops).  Its host-side name is not a device address: the address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that pointer reaches kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
namespace {
std::map<int, void*> g_scratch;   // device -> address of `scratch` (guarded by g_mu)

int scratch_ptr(void** out) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return TQ_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_scratch.find(device);
    if (it == g_scratch.end()) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TQ_EHIP;
        it = g_scratch.emplace(device, ptr).first;
    }
    *out = it->second;
    return TQ_OK;
}
}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_status_string(int status) {
    switch (status) {
        case TQ_OK: return "ok";
        case TQ_EINVAL: return "invalid argument";
        case TQ_EUNSUPPORTED: return "unsupported configuration";
        case TQ_EALIGN: return "device pointer not 16-byte aligned";
        case TQ_EWORKSPACE: return "workspace too small";
        case TQ_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

int tq_get_layout(const tq_params* p, int64_t n_streams, int64_t n_tokens, tq_layout* out) {
    const int rc = check_params(p);
    if (rc != TQ_OK) return rc;
    if (!out || n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    layout_of(p, n_streams, n_tokens, out);
    return TQ_OK;
}

int tq_host_tables(const tq_params* p, int32_t head, double* thresholds, double* centroids, float* signs,
                   float* S) {
    const int rc = check_params(p);
    if (rc != TQ_OK) return rc;
    if (head < 0 || head >= p->n_heads) return TQ_EINVAL;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        const Codebook& cb = codebook(p->d, p->b);
        if (thresholds) std::memcpy(thresholds, cb.thr.data(), cb.thr.size() * 8);
        if (centroids) std::memcpy(centroids, cb.cent.data(), cb.cent.size() * 8);
    }
    if (signs) {
        std::vector<float> s;
        head_signs(p->seed, head, p->d, s);
        std::memcpy(signs, s.data(), p->d * 4);
    }
    if (S && p->m > 0) {
        std::vector<uint16_t> h;
        if (p->sketch == TQ_SKETCH_RHT) rht_matrix_f16(p->seed, head, p->d, h);
        else gaussian_matrix_f16(p->seed, head, p->m, p->d, h);
        for (size_t i = 0; i < h.size(); ++i) S[i] = f16_bits_to_f32(h[i]);
    }
    return TQ_OK;
}

int tq_encode_append(const tq_params* p, const void* x, tq_dtype x_dtype, int64_t n_streams, int64_t n_new,
                     void* packed, int64_t capacity, int64_t t0, void* stream) {
    int rc = check_params(p);
    if (rc != TQ_OK) return rc;
    if (n_streams < 0 || n_new < 0 || capacity < 0 || t0 < 0 || t0 > capacity || n_new > capacity - t0)
        return TQ_EINVAL;
    if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_EINVAL;
    if (n_streams == 0 || n_new == 0) return TQ_OK;
    if (!x || !packed) return TQ_EINVAL;
    if (!aligned16(x) || !aligned16(packed)) return TQ_EALIGN;
    DevTables t;
    int cus = 0;
    if ((rc = get_tables(p, &t, &cus)) != TQ_OK) return rc;
    tq_layout lay;
    layout_of(p, n_streams, capacity, &lay);
    EncodeArgs a{};
    a.x = x;
    a.packed = static_cast<uint8_t*>(packed);
    a.n_streams = n_streams;
    a.n_tokens = n_new;
    a.cap = capacity;
    a.t0 = t0;
    a.off_idx = lay.off_idx;
    a.off_sketch = lay.off_sketch;
    a.off_norm = lay.off_norm;
    a.off_rnorm = lay.off_rnorm;
    a.tiles_per_stream = (n_new + 15) / 16;
    a.n_tiles = n_streams * a.tiles_per_stream;
    a.t = t;
    return hip_status(launch_encode(a, x_dtype == TQ_BF16, cus, static_cast<hipStream_t>(stream)));
}

int tq_encode(const tq_params* p, const void* x, tq_dtype x_dtype, int64_t n_streams, int64_t n_tokens,
              void* packed, void* stream) {
    if (n_tokens < 0) return TQ_EINVAL;
    return tq_encode_append(p, x, x_dtype, n_streams, n_tokens, packed, n_tokens, 0, stream);
}

int tq_encode_kv_append(const tq_params* pk, const tq_params* pv, const void* k, const void* v, tq_dtype x_dtype,
                        int64_t n_streams, int64_t n_new, void* packed_k, void* packed_v, int64_t capacity,
                        int64_t t0, void* stream) {
    int rc = check_params(pk);
    if (rc != TQ_OK) return rc;
    if ((rc = check_params(pv)) != TQ_OK) return rc;
    if (n_streams < 0 || n_new < 0 || capacity < 0 || t0 < 0 || t0 > capacity || n_new > capacity - t0)
        return TQ_EINVAL;
    if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_EINVAL;
    if (n_streams == 0 || n_new == 0) return TQ_OK;
    if (!k || !v || !packed_k || !packed_v) return TQ_EINVAL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(packed_k) || !aligned16(packed_v)) return TQ_EALIGN;
    DevTables tk, tv;
    int cus = 0;
    if ((rc = get_tables(pk, &tk, &cus)) != TQ_OK) return rc;
    if ((rc = get_tables(pv, &tv, &cus)) != TQ_OK) return rc;
    auto args = [&](const tq_params* p, const DevTables& t, const void* x, void* packed) {
        tq_layout lay;
        layout_of(p, n_streams, capacity, &lay);
        EncodeArgs a{};
        a.x = x;
        a.packed = static_cast<uint8_t*>(packed);
        a.n_streams = n_streams;
        a.n_tokens = n_new;
        a.cap = capacity;
        a.t0 = t0;
        a.off_idx = lay.off_idx;
        a.off_sketch = lay.off_sketch;
        a.off_norm = lay.off_norm;
        a.off_rnorm = lay.off_rnorm;
        a.tiles_per_stream = (n_new + 15) / 16;
        a.n_tiles = n_streams * a.tiles_per_stream;
        a.t = t;
        return a;
    };
    const EncodeArgs ak = args(pk, tk, k, packed_k), av = args(pv, tv, v, packed_v);
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool fused = false;
    if (x_dtype == TQ_BF16) {
        rc = hip_status(launch_encode_kv(ak, av, cus, s, &fused));
        if (rc != TQ_OK || fused) return rc;
    }
    if ((rc = hip_status(launch_encode(ak, x_dtype == TQ_BF16, cus, s))) != TQ_OK) return rc;
    return hip_status(launch_encode(av, x_dtype == TQ_BF16, cus, s));
}

int tq_encode_kv(const tq_params* pk, const tq_params* pv, const void* k, const void* v, tq_dtype x_dtype,
                 int64_t n_streams, int64_t n_tokens, void* packed_k, void* packed_v, void* stream) {
    if (n_tokens < 0) return TQ_EINVAL;
    return tq_encode_kv_append(pk, pv, k, v, x_dtype, n_streams, n_tokens, packed_k, packed_v, n_tokens, 0, stream);
}

int tq_decode(const tq_params* p, const void* packed, int64_t n_streams, int64_t n_tokens, void* x_hat,
              tq_dtype out_dtype, void* stream) {
    int rc = check_params(p);
    if (rc != TQ_OK) return rc;
    if (n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0) return TQ_OK;
    if (!x_hat || !packed) return TQ_EINVAL;
    if (!aligned16(x_hat) || !aligned16(packed)) return TQ_EALIGN;
    DevTables t;
    int cus = 0;
    if ((rc = get_tables(p, &t, &cus)) != TQ_OK) return rc;
    tq_layout lay;
    layout_of(p, n_streams, n_tokens, &lay);
    DecodeArgs a{};
    a.packed = static_cast<const uint8_t*>(packed);
    a.out = x_hat;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.off_idx = lay.off_idx;
    a.off_norm = lay.off_norm;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    a.n_tiles = n_streams * a.tiles_per_stream;
    a.t = t;
    return hip_status(launch_decode(a, out_dtype == TQ_BF16, cus, static_cast<hipStream_t>(stream)));
}

int tq_decode_qjl(const tq_params* p, const void* packed, int64_t n_streams, int64_t n_tokens, void* x_hat,
                  tq_dtype out_dtype, void* stream) {
    int rc = check_params(p);
    if (rc != TQ_OK) return rc;
    if (p->m == 0) return TQ_EINVAL;
    if (n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0) return TQ_OK;
    if (!x_hat || !packed) return TQ_EINVAL;
    if (!aligned16(x_hat) || !aligned16(packed)) return TQ_EALIGN;
    DevTables t;
    int cus = 0;
    if ((rc = get_tables(p, &t, &cus)) != TQ_OK) return rc;
    tq_layout lay;
    layout_of(p, n_streams, n_tokens, &lay);
    DecodeArgs a{};
    a.packed = static_cast<const uint8_t*>(packed);
    a.out = x_hat;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.off_idx = lay.off_idx;
    a.off_norm = lay.off_norm;
    a.off_sketch = lay.off_sketch;
    a.off_rnorm = lay.off_rnorm;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    a.n_tiles = n_streams * a.tiles_per_stream;
    a.t = t;
    bool supported = true;
    const hipError_t e = launch_decode_qjl(a, out_dtype == TQ_BF16, cus, static_cast<hipStream_t>(stream), &supported);
    if (!supported) return TQ_EUNSUPPORTED;
    return hip_status(e);
}

size_t tq_scores_workspace_bytes(const tq_params* pk, int64_t n_streams, int64_t n_q) {
    if (check_params(pk) != TQ_OK || n_streams < 0 || n_q < 0) return 0;
    return (size_t)qops_layout(0, n_streams * n_q + 16, pk->d, pk->m).end;
}

int tq_qk_scores(const tq_params* pk, const void* q, tq_dtype q_dtype, int64_t n_q, const void* packed_k,
                 int64_t n_streams, int64_t n_tokens, float* scores, void* workspace, size_t workspace_bytes,
                 void* stream) {
    int rc = check_params(pk);
    if (rc != TQ_OK) return rc;
    if (n_streams < 0 || n_tokens < 0 || n_q < 0 || n_q > 256) return TQ_EINVAL;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0 || n_q == 0) return TQ_OK;
    if (!q || !packed_k || !scores || !workspace) return TQ_EINVAL;
    if (!aligned16(q) || !aligned16(packed_k) || !aligned16(scores) || !aligned16(workspace)) return TQ_EALIGN;
    if (workspace_bytes < tq_scores_workspace_bytes(pk, n_streams, n_q)) return TQ_EWORKSPACE;
    DevTables t;
    int cus = 0;
    if ((rc = get_tables(pk, &t, &cus)) != TQ_OK) return rc;
    tq_layout lay;
    layout_of(pk, n_streams, n_tokens, &lay);
    const QOps qo = qops_at(static_cast<uint8_t*>(workspace), qops_layout(0, n_streams * n_q + 16, pk->d, pk->m));
    hipStream_t s = static_cast<hipStream_t>(stream);
    QPrepArgs qa{};
    qa.q = q;
    qa.q_bf16 = q_dtype == TQ_BF16;
    qa.n_rows = n_streams * n_q;
    qa.n_q_per_stream = (int)n_q;
    qa.q_scale = 1.0f;
    qa.p_scale = 1.0f;
    qa.o = qo;
    qa.t = t;
    if ((rc = hip_status(launch_qprep(qa, s))) != TQ_OK) return rc;
    ScoresArgs a{};
    a.packed = static_cast<const uint8_t*>(packed_k);
    a.o = qo;
    a.scores = scores;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.n_q = (int)n_q;
    a.off_idx = lay.off_idx;
    a.off_sketch = lay.off_sketch;
    a.off_norm = lay.off_norm;
    a.off_rnorm = lay.off_rnorm;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    a.n_tiles = n_streams * a.tiles_per_stream;
    a.t = t;
    return hip_status(launch_scores(a, cus, s));
}

size_t tq_attention_workspace_bytes(const tq_params* pk, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int64_t n_tokens) {
    if (check_params(pk) != TQ_OK || batch < 0 || n_q_heads < 0 || n_kv_heads < 1 || n_tokens < 0) return 0;
    return (size_t)attn_ws(pk, batch, n_q_heads, n_kv_heads, n_tokens).total;
}

int tq_decode_attention(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype, int32_t batch,
                        int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k, const void* packed_v,
                        int64_t n_tokens, float softmax_scale, void* out, tq_dtype out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return tq_decode_attention_varlen(pk, pv, q, q_dtype, batch, n_q_heads, n_kv_heads, packed_k, packed_v, n_tokens,
                                      nullptr, softmax_scale, out, out_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace tq {
namespace {
// decode-attention on a given workspace; `no_alloc`: find the tables instead of building them
int attention_impl(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype, int32_t batch,
                   int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k, const void* packed_v,
                   int64_t n_tokens, const int32_t* lengths, float softmax_scale, void* out, tq_dtype out_dtype,
                   void* workspace, size_t workspace_bytes, void* stream, bool no_alloc) {
    int rc = check_params(pk);
    if (rc != TQ_OK) return rc;
    if ((rc = check_params(pv)) != TQ_OK) return rc;
    if (pv->m != 0 || pk->d != pv->d) return TQ_EINVAL;
    if (batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_tokens < 0) return TQ_EINVAL;
    if (n_q_heads % n_kv_heads != 0 || n_q_heads / n_kv_heads > 16) return TQ_EINVAL;
    if (pk->n_heads != n_kv_heads || pv->n_heads != n_kv_heads) return TQ_EINVAL;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_EINVAL;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_EINVAL;
    if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale)) return TQ_EINVAL;
    if (batch == 0) return TQ_OK;
    if (n_tokens == 0) return TQ_EINVAL;  // softmax over an empty cache is undefined
    if (!q || !packed_k || !packed_v || !out || !workspace) return TQ_EINVAL;
    if (!aligned16(q) || !aligned16(packed_k) || !aligned16(packed_v) || !aligned16(out) || !aligned16(workspace))
        return TQ_EALIGN;
    if (lengths && (reinterpret_cast<uintptr_t>(lengths) & 3u)) return TQ_EALIGN;
    const AttnWs w = attn_ws(pk, batch, n_q_heads, n_kv_heads, n_tokens);
    if (workspace_bytes < (size_t)w.total) return TQ_EWORKSPACE;
    if (!attention_supported(pk->d, pk->b, pv->b)) return TQ_EUNSUPPORTED;
    // the kernel addresses a stream's planes with 32-bit offsets (the index planes are the largest)
    const int64_t max_row = std::max<int64_t>(pk->d * pk->b / 8, pv->d * pv->b / 8);
    if (n_tokens > (int64_t)((1ull << 32) - (1ull << 16)) / max_row) return TQ_EUNSUPPORTED;
    DevTables tk, tv;
    int cus = 0;
    if ((rc = (no_alloc ? find_tables : get_tables)(pk, &tk, &cus)) != TQ_OK) return rc;
    if ((rc = (no_alloc ? find_tables : get_tables)(pv, &tv, &cus)) != TQ_OK) return rc;
    const int64_t streams = (int64_t)batch * n_kv_heads;
    tq_layout lk, lv;
    layout_of(pk, streams, n_tokens, &lk);
    layout_of(pv, streams, n_tokens, &lv);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    QPrepArgs qa{};
    qa.q = q;
    qa.q_bf16 = q_dtype == TQ_BF16;
    qa.n_rows = (int64_t)batch * n_q_heads;
    qa.n_q_per_stream = n_q_heads / n_kv_heads;
    qa.o = qops_at(ws, w.q);
    qa.t = tk;
    // the attention kernel works with base-2 logits: fold scale·log2(e) into the rotated queries
    // and scale·log2(e)·sqrt(pi/2)/m into their sketch projections
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)pk->d);
    const float scale_log2 = scale * 1.4426950408889634f;
    qa.q_scale = scale_log2;
    qa.p_scale = pk->m > 0 ? scale_log2 * (float)(std::sqrt(M_PI / 2.0) / pk->m) : 0.0f;
    AttnArgs a{};
    a.pk = static_cast<const uint8_t*>(packed_k);
    a.pv = static_cast<const uint8_t*>(packed_v);
    a.o = qa.o;
    a.part = reinterpret_cast<float*>(ws + w.o_part);
    a.part_ml = reinterpret_cast<float*>(ws + w.o_ml);
    a.out = out;
    a.out_bf16 = out_dtype == TQ_BF16;
    a.n_tokens = n_tokens;
    a.lens = lengths;
    a.batch = batch;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.group = n_q_heads / n_kv_heads;
    a.n_split = (int)w.n_split;
    a.tokens_per_split = attn_tokens_per_split(pk->d, pk->b, a.group, streams, n_tokens);
    a.scale_log2 = scale_log2;
    a.k_off_idx = lk.off_idx;
    a.k_off_sketch = lk.off_sketch;
    a.k_off_norm = lk.off_norm;
    a.k_off_rnorm = lk.off_rnorm;
    a.v_off_idx = lv.off_idx;
    a.v_off_norm = lv.off_norm;
    a.tk = tk;
    a.tv = tv;
    a.q = q;
    a.q_bf16 = qa.q_bf16;
    a.q_scale = qa.q_scale;
    a.p_scale = qa.p_scale;
    // the query prep runs inside the attention kernel where every block covers one stream, else as
    // its own launch writing the workspace's query operands
    a.fused_q = attention_fuses_qprep(a) ? 1 : 0;
    if (!a.fused_q && (rc = hip_status(launch_qprep(qa, s))) != TQ_OK) return rc;
    bool supported = true;
    const hipError_t e = launch_attention(a, cus, s, &supported);
    if (!supported) return TQ_EUNSUPPORTED;
    return hip_status(e);
}
}  // namespace
}  // namespace tq

extern "C" {

int tq_decode_attention_varlen(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype,
                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                               const void* packed_v, int64_t n_tokens, const int32_t* lengths, float softmax_scale,
                               void* out, tq_dtype out_dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return attention_impl(pk, pv, q, q_dtype, batch, n_q_heads, n_kv_heads, packed_k, packed_v, n_tokens, lengths,
                          softmax_scale, out, out_dtype, workspace, workspace_bytes, stream, false);
}

size_t tq_attention_noalloc_max_bytes(void) { return kScratchBytes; }

int tq_decode_attention_noalloc(const tq_params* pk, const tq_params* pv, const void* q, tq_dtype q_dtype,
                                int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                                const void* packed_v, int64_t n_tokens, const int32_t* lengths,
                                float softmax_scale, void* out, tq_dtype out_dtype, void* stream) {
    int rc = check_params(pk);
    if (rc != TQ_OK) return rc;
    if (batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_tokens < 0) return TQ_EINVAL;
    // the scratch array bounds the workspace: larger problems are rejected before any device call
    if (tq_attention_workspace_bytes(pk, batch, n_q_heads, n_kv_heads, n_tokens) > kScratchBytes) return TQ_EWORKSPACE;
    void* ws = nullptr;
    if ((rc = scratch_ptr(&ws)) != TQ_OK) return rc;
    return attention_impl(pk, pv, q, q_dtype, batch, n_q_heads, n_kv_heads, packed_k, packed_v, n_tokens, lengths,
                          softmax_scale, out, out_dtype, ws, kScratchBytes, stream, true);
}

void tq_clear_cache(void) {
    {
        std::lock_guard<std::mutex> lk(g_mu);
        for (auto& kv : g_tables) (void)hipFree(kv.second.blob);
        g_tables.clear();
    }
    fmag_clear_tables();
}

}  // extern "C"
