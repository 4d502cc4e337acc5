// SpectralQuant codec, host side: calibration (covariance, Jacobi eigensolver, effective dimension,
// bit allocation), the Gaussian Lloyd-Max codebooks, the device tables, and the C ABI of
// include/tq_sq.h.  "Ablation, Statistical Inference, and Validation for KV-Cache Compression",
// §2 "SpectralQuant", §6 "Water-filling", §7 "Spectral gap criterion".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <numeric>
#include <vector>

#include "../../include/tq_sq.h"
#include "sq_kernels.hpp"
#include "tables.hpp"

struct tq_sq_codec {
    tq::SqDev dev;
    int device = 0;
    int num_cus = 0;
};

namespace tq {
namespace {

constexpr int kBMax = 8;
constexpr double kLambdaFloor = 1e-12;

// ---- Gaussian Lloyd-Max ([MAX] J. Max 1960): positive half, Lloyd sweeps then Newton ----------
double upper_q(double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x / std::sqrt(2.0)); }
double phi(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

void gauss_lloyd_max(int b, std::vector<double>& thr, std::vector<double>& cent) {
    const int L = 1 << b, K = L / 2;
    std::vector<double> c(K), t(K + 1), cn(K);
    for (int k = 0; k < K; ++k) {  // start at the quantiles (K + k + 1/2)/L, by bisection on erfc
        const double p = (K + k + 0.5) / L;
        double lo = -10, hi = 10;
        for (int it = 0; it < 200; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (1.0 - upper_q(mid) < p) lo = mid; else hi = mid;
        }
        c[k] = 0.5 * (lo + hi);
    }
    auto edges = [&]() {
        t[0] = 0.0;
        t[K] = std::numeric_limits<double>::infinity();
        for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    };
    for (int it = 0; it < 200000; ++it) {
        edges();
        double delta = 0.0;
        for (int k = 0; k < K; ++k) {
            cn[k] = (phi(t[k]) - phi(t[k + 1])) / (upper_q(t[k]) - upper_q(t[k + 1]));
            delta = std::max(delta, std::fabs(cn[k] - c[k]));
        }
        c.swap(cn);
        if (delta < 1e-7 || K == 1) break;
    }
    if (K > 1) {  // Newton on R_k = c_k·mass_k - moment_k (tridiagonal Jacobian)
        std::vector<double> mass(K), R(K), lo(K), di(K), up(K), cp(K), dp(K), dc(K);
        for (int it = 0; it < 100; ++it) {
            edges();
            for (int k = 0; k < K; ++k) {
                mass[k] = upper_q(t[k]) - upper_q(t[k + 1]);
                R[k] = c[k] * mass[k] - (phi(t[k]) - phi(t[k + 1]));
                const double dlo = (k > 0) ? (t[k] - c[k]) * phi(t[k]) : 0.0;
                const double dhi = (k + 1 < K) ? (c[k] - t[k + 1]) * phi(t[k + 1]) : 0.0;
                di[k] = mass[k] + 0.5 * dlo + 0.5 * dhi;
                lo[k] = 0.5 * dlo;
                up[k] = 0.5 * dhi;
            }
            cp[0] = up[0] / di[0];
            dp[0] = -R[0] / di[0];
            for (int k = 1; k < K; ++k) {
                const double den = di[k] - lo[k] * cp[k - 1];
                cp[k] = up[k] / den;
                dp[k] = (-R[k] - lo[k] * dp[k - 1]) / den;
            }
            dc[K - 1] = dp[K - 1];
            for (int k = K - 2; k >= 0; --k) dc[k] = dp[k] - cp[k] * dc[k + 1];
            double step = 0.0;
            for (int k = 0; k < K; ++k) {
                c[k] += dc[k];
                step = std::max(step, std::fabs(dc[k]) / std::fabs(c[k]));
            }
            if (step < 1e-16) break;
        }
    }
    cent.assign(L, 0.0);
    thr.assign(L - 1, 0.0);
    for (int k = 0; k < K; ++k) {
        cent[K + k] = c[k];
        cent[K - 1 - k] = -c[k];
    }
    for (int k = 0; k < L - 1; ++k) thr[k] = 0.5 * (cent[k] + cent[k + 1]);
}

struct GaussBook {
    std::vector<double> thr, cent;
};
std::mutex g_sq_mu;
const GaussBook& gauss_book(int b) {
    static std::map<int, GaussBook> books;
    std::lock_guard<std::mutex> lk(g_sq_mu);
    auto it = books.find(b);
    if (it == books.end()) {
        GaussBook g;
        gauss_lloyd_max(b, g.thr, g.cent);
        it = books.emplace(b, std::move(g)).first;
    }
    return it->second;
}

// ---- symmetric eigensolver: cyclic Jacobi rotations (Golub & Van Loan §8.5) -------------------
// A (n x n, row-major) is destroyed; on return w holds the eigenvalues and V (row-major) the
// eigenvectors as columns.
void jacobi_eigh(std::vector<double>& A, int n, std::vector<double>& w, std::vector<double>& V) {
    V.assign((size_t)n * n, 0.0);
    for (int i = 0; i < n; ++i) V[(size_t)i * n + i] = 1.0;
    auto a = [&](int i, int j) -> double& { return A[(size_t)i * n + j]; };
    for (int sweep = 0; sweep < 100; ++sweep) {
        double off = 0.0, tot = 0.0;
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) (i == j ? tot : off) += a(i, j) * a(i, j);
        if (off <= 1e-32 * (tot + off) || off == 0.0) break;
        for (int p = 0; p < n - 1; ++p)
            for (int q = p + 1; q < n; ++q) {
                const double apq = a(p, q);
                if (apq == 0.0) continue;
                const double theta = (a(q, q) - a(p, p)) / (2.0 * apq);
                const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
                const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
                for (int k = 0; k < n; ++k) {  // columns p, q
                    const double akp = a(k, p), akq = a(k, q);
                    a(k, p) = c * akp - s * akq;
                    a(k, q) = s * akp + c * akq;
                }
                for (int k = 0; k < n; ++k) {  // rows p, q
                    const double apk = a(p, k), aqk = a(q, k);
                    a(p, k) = c * apk - s * aqk;
                    a(q, k) = s * apk + c * aqk;
                }
                for (int k = 0; k < n; ++k) {
                    double& vkp = V[(size_t)k * n + p];
                    double& vkq = V[(size_t)k * n + q];
                    const double x = vkp, y = vkq;
                    vkp = c * x - s * y;
                    vkq = s * x + c * y;
                }
            }
    }
    w.resize(n);
    for (int i = 0; i < n; ++i) w[i] = a(i, i);
}

int effective_dim(const std::vector<double>& lam, double gamma, int d_eff_max) {
    const int d = (int)lam.size();
    double s = 0.0, s2 = 0.0;
    for (double l : lam) {
        s += l;
        s2 += l * l;
    }
    int d_eff = s2 > 0.0 ? (int)std::floor(s * s / s2 + 0.5) : 1;
    d_eff = std::min(std::max(d_eff, 1), d);
    if (gamma > 0.0)
        for (int k = 1; k < d_eff; ++k)
            if (lam[k] <= 0.0 || lam[k - 1] / lam[k] > gamma) {
                d_eff = k;
                break;
            }
    if (d_eff_max > 0) d_eff = std::min(d_eff, d_eff_max);
    return std::max(d_eff, 1);
}

std::vector<double> floored(const double* lam, int d) {
    std::vector<double> o(lam, lam + d);
    if (!(lam[0] > 0.0)) {
        std::fill(o.begin(), o.end(), 1.0);
        return o;
    }
    for (double& v : o) v = std::max(v, kLambdaFloor * lam[0]);
    return o;
}

// greedy integer water-filling of Σ λ_k 4^-b_k, Σ b_k = total, b_tail <= b_k <= 8
void waterfill(const std::vector<double>& lam, int n, int total, int b_tail, int32_t* bits) {
    for (int k = 0; k < n; ++k) bits[k] = b_tail;
    for (int left = total - n * b_tail; left > 0; --left) {
        int best = -1;
        double bv = 0.0;
        for (int k = 0; k < n; ++k) {
            if (bits[k] >= kBMax) continue;
            const double v = lam[k] * std::ldexp(1.0, -2 * bits[k]);
            if (best < 0 || v > bv || (v == bv && bits[k] < bits[best])) {
                best = k;
                bv = v;
            }
        }
        if (best < 0) break;
        ++bits[best];
    }
}

int check_sq_params(const tq_sq_params* p, bool kernels) {
    if (!p) return TQ_EINVAL;
    if (kernels ? (p->d != 64 && p->d != 128) : (p->d != 64 && p->d != 128 && p->d != 256)) return TQ_EINVAL;
    if (p->n_heads < 1) return TQ_EINVAL;
    return TQ_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// the codec's tables live on one device, which must be the current one
bool on_codec_device(const tq_sq_codec* c) {
    int cur = -1;
    return hipGetDevice(&cur) == hipSuccess && cur == c->device;
}

struct Blob {
    std::vector<uint8_t> host;
    int64_t add(const void* src, int64_t bytes) {
        const int64_t off = (int64_t)((host.size() + 255) / 256 * 256);
        host.resize(off + (bytes + 255) / 256 * 256);
        std::memcpy(host.data() + off, src, bytes);
        return off;
    }
};

// attention split geometry, a function of the arguments only: about as many (stream, split) waves
// as 256 CUs hold at eight per CU, splits of at least 256 tokens in multiples of 32, at most 1024
struct SqAttnWs {
    int64_t tps, n_split, o_qs, o_pp, o_ps, o_ql, o_part, o_ml, total;
};
SqAttnWs sq_attn_ws(int d, int m, int64_t streams, int64_t n_tokens) {
    SqAttnWs w{};
    int64_t ns = (256 * 8 + streams - 1) / (streams > 0 ? streams : 1);
    ns = std::min(ns, (n_tokens + 255) / 256);
    ns = std::max<int64_t>(std::min<int64_t>(ns, 1024), 1);
    w.tps = std::max<int64_t>(((n_tokens + ns - 1) / ns + 31) / 32 * 32, 32);
    w.n_split = std::max<int64_t>((n_tokens + w.tps - 1) / w.tps, 1);
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    w.o_qs = al(streams * 16 * d * 2);
    w.o_pp = w.o_qs + al(streams * 16 * 4);          // with a key sketch: S q_Z rows (64 fp16) and scales
    w.o_ps = w.o_pp + (m > 0 ? al(streams * 16 * 64 * 2) : 0);
    w.o_ql = w.o_ps + (m > 0 ? al(streams * 16 * 4) : 0);   // the fp16 remainders of the projected queries
    w.o_part = w.o_ql + al(streams * 16 * d * 2);
    w.o_ml = w.o_part + al(streams * w.n_split * 16 * d * 4);
    w.total = w.o_ml + al(streams * w.n_split * 16 * 2 * 4);
    return w;
}

void split_f16(double v, uint16_t* hi, uint16_t* lo) {
    *hi = f64_to_f16_bits(v);
    *lo = f64_to_f16_bits(v - (double)f16_bits_to_f32(*hi));
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

int tq_sq_calibrate(const tq_sq_params* p, const float* x_cal, int64_t n_cal, double* basis,
                    double* lambda, int32_t* bits, int32_t* d_eff) {
    if (check_sq_params(p, false) != TQ_OK || !x_cal || n_cal < 1) return TQ_EINVAL;
    if (p->b < 1 || p->b > kBMax || p->b_tail < 1 || p->b_tail > p->b) return TQ_EINVAL;
    if (p->d_eff_max < 0) return TQ_EINVAL;
    const int d = p->d;
    std::vector<double> C((size_t)d * d), w, V, Vs((size_t)d * d);
    for (int h = 0; h < p->n_heads; ++h) {
        const float* X = x_cal + (size_t)h * n_cal * d;
        std::fill(C.begin(), C.end(), 0.0);
        for (int64_t r = 0; r < n_cal; ++r) {
            const float* xr = X + (size_t)r * d;
            for (int i = 0; i < d; ++i) {
                const double xi = xr[i];
                double* ci = &C[(size_t)i * d];
                for (int j = i; j < d; ++j) ci[j] += xi * (double)xr[j];
            }
        }
        for (int i = 0; i < d; ++i)
            for (int j = i; j < d; ++j) {
                C[(size_t)i * d + j] /= (double)n_cal;
                C[(size_t)j * d + i] = C[(size_t)i * d + j];
            }
        jacobi_eigh(C, d, w, V);
        std::vector<int> order(d);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] > w[b]; });
        std::vector<double> lam(d);
        for (int k = 0; k < d; ++k) {
            const int src = order[k];
            lam[k] = w[src];
            int piv = 0;  // canonical sign: the first entry of largest magnitude is positive
            for (int j = 1; j < d; ++j)
                if (std::fabs(V[(size_t)j * d + src]) > std::fabs(V[(size_t)piv * d + src])) piv = j;
            const double sg = V[(size_t)piv * d + src] < 0 ? -1.0 : 1.0;
            for (int j = 0; j < d; ++j) Vs[(size_t)j * d + k] = sg * V[(size_t)j * d + src];
        }
        const int de = effective_dim(lam, p->gamma, p->d_eff_max);
        std::vector<int32_t> bh(d, p->b_tail);
        const std::vector<double> lc = floored(lam.data(), d);
        if (p->waterfill) waterfill(lc, de, p->b * de, p->b_tail, bh.data());
        else for (int k = 0; k < de; ++k) bh[k] = p->b;
        if (basis) std::memcpy(basis + (size_t)h * d * d, Vs.data(), sizeof(double) * d * d);
        if (lambda) std::memcpy(lambda + (size_t)h * d, lam.data(), sizeof(double) * d);
        if (bits) std::memcpy(bits + (size_t)h * d, bh.data(), sizeof(int32_t) * d);
        if (d_eff) d_eff[h] = de;
    }
    return TQ_OK;
}

int tq_sq_create(const tq_sq_params* p, const double* basis, const double* lambda, const int32_t* bits,
                 const int32_t* d_eff, tq_sq_codec** out) {
    if (check_sq_params(p, true) != TQ_OK || !basis || !lambda || !bits || !out) return TQ_EINVAL;
    const int d = p->d, H = p->n_heads, T = d / 16, S = d / 32, M = p->m;
    if (M != 0 && M != 16 && M != 32 && M != 48 && M != 64) return TQ_EINVAL;
    if (M > 0) {
        if (!d_eff) return TQ_EINVAL;
        for (int h = 0; h < H; ++h) {
            if (d_eff[h] < 1 || d_eff[h] > d) return TQ_EINVAL;
            if (d_eff[h] > 32) return TQ_EUNSUPPORTED;
        }
    }
    for (int64_t i = 0; i < (int64_t)H * d * d; ++i)
        if (!std::isfinite(basis[i])) return TQ_EINVAL;
    for (int64_t i = 0; i < (int64_t)H * d; ++i) {
        if (!std::isfinite(lambda[i])) return TQ_EINVAL;
        if (bits[i] < 1 || bits[i] > kBMax) return TQ_EINVAL;
    }
    // grids of the widths in use
    bool used[kBMax + 1] = {};
    for (int64_t i = 0; i < (int64_t)H * d; ++i) used[bits[i]] = true;
    std::vector<uint32_t> grids;
    int goff[kBMax + 1] = {}, gG[kBMax + 1] = {};
    for (int w = 1; w <= kBMax; ++w) {
        if (!used[w]) continue;
        const GaussBook& gb = gauss_book(w);
        std::vector<double> ty(gb.thr.size());
        for (size_t i = 0; i < ty.size(); ++i) ty[i] = gb.thr[i] / kSqRange;
        Grid g;
        if (!build_grid(ty, g)) return TQ_EUNSUPPORTED;
        goff[w] = (int)(grids.size() / 2);
        gG[w] = g.G;
        grids.insert(grids.end(), g.entries.begin(), g.entries.end());
    }
    // codebooks of every width w at rows w·256 (row 0 unused): (hi, lo) of c·2^12 and fp16 c
    std::vector<uint16_t> cb_hl(2 * 256 * (kBMax + 1), 0), cb_h(256 * (kBMax + 1), 0);
    for (int w = 1; w <= kBMax; ++w) {
        const GaussBook& gb = gauss_book(w);
        for (int i = 0; i < (1 << w); ++i) {
            const int e = w * 256 + i;
            split_f16(gb.cent[i] * 4096.0, &cb_hl[2 * e], &cb_hl[2 * e + 1]);
            cb_h[e] = f64_to_f16_bits(gb.cent[i]);
        }
    }
    int max_bits = 0;
    for (int h = 0; h < H; ++h) {
        int s = 0;
        for (int k = 0; k < d; ++k) s += bits[(size_t)h * d + k];
        max_bits = std::max(max_bits, s);
    }
    const int rec_words = (max_bits + (M > 0 ? M + 16 : 0) + 31) / 32;

    std::vector<uint16_t> enc_b((size_t)H * 2 * T * S * 512), dec_a((size_t)H * 2 * T * S * 512);
    std::vector<float> desc((size_t)H * d * 4), dscale(H), U32((size_t)H * d * d), sig((size_t)H * d);
    std::vector<uint32_t> fields((size_t)H * S * 4 * 4);
    for (int h = 0; h < H; ++h) {
        const double* U = basis + (size_t)h * d * d;
        const int32_t* bh = bits + (size_t)h * d;
        const std::vector<double> lc = floored(lambda + (size_t)h * d, d);
        std::vector<double> sg(d);
        std::vector<int> off(d + 1, 0);
        for (int k = 0; k < d; ++k) {
            sg[k] = std::sqrt(lc[k]);
            off[k + 1] = off[k] + bh[k];
            sig[(size_t)h * d + k] = (float)sg[k];
        }
        for (int j = 0; j < d; ++j)
            for (int k = 0; k < d; ++k) U32[((size_t)h * d + j) * d + k] = (float)U[(size_t)j * d + k];
        // encode B operand: B[kk = 8g + i][n = lane % 16] of (tile t, kstep s) = U[32 s + 8 g + i][16 t + n] · 2^8
        for (int t = 0; t < T; ++t)
            for (int s = 0; s < S; ++s)
                for (int l = 0; l < 64; ++l)
                    for (int i = 0; i < 8; ++i) {
                        const double v = U[(size_t)(32 * s + 8 * (l / 16) + i) * d + 16 * t + (l % 16)] * 256.0;
                        uint16_t hi, lo;
                        split_f16(v, &hi, &lo);
                        const size_t base = ((((size_t)h * 2 + 0) * T + t) * S + s) * 512 + l * 8 + i;
                        enc_b[base] = hi;
                        enc_b[base + (size_t)T * S * 512] = lo;
                    }
        // encode per-dimension descriptor: u_grid = (acc · 2^-sc) · mul + add with acc = 2^(8+sc) z
        // and add = G/2 + 1 (cells clamp to [0, 2·add]); meta = grid offset | bit offset << 16 |
        // width << 26; meta2 = the field's bit position within its group of 4 dimensions 4q..4q+3
        for (int k = 0; k < d; ++k) {
            const int w = bh[k], G = gG[w], kq = k & ~3;
            float* o = &desc[((size_t)h * d + k) * 4];
            o[0] = (float)(std::ldexp(1.0, -8) * (G / (2.0 * kSqRange)) / sg[k]);
            o[1] = (float)(0.5 * G + 1.0);
            const uint32_t meta = (uint32_t)goff[w] | ((uint32_t)off[k] << 16) | ((uint32_t)w << 26);
            const uint32_t meta2 = (uint32_t)(off[k] - off[kq]);
            std::memcpy(&o[2], &meta, 4);
            std::memcpy(&o[3], &meta2, 4);
        }
        // decode A operand: A[m = lane % 16][kk = 8 g + i] of (tile t, kstep s) = U[16 t + m][32 s + 8 g + i] σ · 2^e
        double mx = 0.0;
        for (int j = 0; j < d; ++j)
            for (int k = 0; k < d; ++k) mx = std::max(mx, std::fabs(U[(size_t)j * d + k] * sg[k]));
        const int e = mx > 0 ? 13 - (int)std::floor(std::log2(mx)) : 0;
        dscale[h] = (float)std::ldexp(1.0, -(e + 12));
        for (int t = 0; t < T; ++t)
            for (int s = 0; s < S; ++s)
                for (int l = 0; l < 64; ++l)
                    for (int i = 0; i < 8; ++i) {
                        const int j = 16 * t + (l % 16), k = 32 * s + 8 * (l / 16) + i;
                        uint16_t hi, lo;
                        split_f16(std::ldexp(U[(size_t)j * d + k] * sg[k], e), &hi, &lo);
                        const size_t base = ((((size_t)h * 2 + 0) * T + t) * S + s) * 512 + l * 8 + i;
                        dec_a[base] = hi;
                        dec_a[base + (size_t)T * S * 512] = lo;
                    }
        // field extraction of the 8 fields k = 32 s + 8 g + i: they lie in the 64 bits from bit
        // off[k0] = 32 w0 + r0 of the record; {w0 | r0 << 8, positions of fields 1..4 and 5..7
        // within those 64 bits (8 bits each), widths (4 bits each)}
        for (int s = 0; s < S; ++s)
            for (int g = 0; g < 4; ++g) {
                const int k0 = 32 * s + 8 * g, w0 = off[k0] >> 5, r0 = off[k0] & 31;
                uint32_t p14 = 0, p57 = 0, wid = 0;
                for (int i = 0; i < 8; ++i) {
                    const uint32_t pos = (uint32_t)(off[k0 + i] - off[k0]);
                    if (i >= 1 && i <= 4) p14 |= pos << (8 * (i - 1));
                    if (i >= 5) p57 |= pos << (8 * (i - 5));
                    wid |= (uint32_t)bh[k0 + i] << (4 * i);
                }
                uint32_t* f = &fields[(((size_t)h * S + s) * 4 + g) * 4];
                f[0] = (uint32_t)w0 | ((uint32_t)r0 << 8);
                f[1] = p14;
                f[2] = p57;
                f[3] = wid;
            }
    }

    // the selective QJL sketch
    std::vector<uint16_t> skb(M > 0 ? (size_t)H * (M / 16) * 512 : 1, 0);
    std::vector<float> sk32(M > 0 ? (size_t)H * 64 * 32 : 1, 0.0f), cent32(256 * (kBMax + 1), 0.0f);
    std::vector<int32_t> skoff(H, 0), deffv(H, 0);
    std::vector<uint16_t> pm1(256 * 8);
    for (int v = 0; v < 256; ++v)
        for (int i = 0; i < 8; ++i) pm1[v * 8 + i] = ((v >> i) & 1) ? 0x3c00u : 0xbc00u;   // fp16 +1, -1
    for (int w = 1; w <= kBMax; ++w) {
        const GaussBook& gb = gauss_book(w);
        for (int i = 0; i < (1 << w); ++i) cent32[w * 256 + i] = (float)gb.cent[i];
    }
    for (int h = 0; h < H; ++h) {
        int sb = 0;
        for (int k = 0; k < d; ++k) sb += bits[(size_t)h * d + k];
        skoff[h] = sb;
        deffv[h] = d_eff ? d_eff[h] : 0;
        if (M == 0) continue;
        const uint64_t key = stream_key(p->seed, 4, (uint32_t)h);
        auto sgn = [&](int i, int k) {   // S[i][k] = -1 iff bit 63 of word i·d + k
            return (mix64(key + (uint64_t)(i * d + k + 1) * 0x9E3779B97F4A7C15ull) >> 63) ? -1.0f : 1.0f;
        };
        for (int i = 0; i < M; ++i)
            for (int k = 0; k < d_eff[h]; ++k) sk32[((size_t)h * 64 + i) * 32 + k] = sgn(i, k);
        for (int ts = 0; ts < M / 16; ++ts)
            for (int l = 0; l < 64; ++l)
                for (int i = 0; i < 8; ++i) {   // B[kk = 8 g + i][n = l % 16] = S[16 ts + n][8 g + i]
                    const float v = sk32[((size_t)h * 64 + 16 * ts + (l % 16)) * 32 + 8 * (l / 16) + i];
                    skb[(((size_t)h * (M / 16) + ts) * 64 + l) * 8 + i] = f64_to_f16_bits(v);
                }
    }

    Blob blob;
    const int64_t o_skb = blob.add(skb.data(), skb.size() * 2);
    const int64_t o_sk32 = blob.add(sk32.data(), sk32.size() * 4);
    const int64_t o_c32 = blob.add(cent32.data(), cent32.size() * 4);
    const int64_t o_skoff = blob.add(skoff.data(), skoff.size() * 4);
    const int64_t o_deff = blob.add(deffv.data(), deffv.size() * 4);
    const int64_t o_pm1 = blob.add(pm1.data(), pm1.size() * 2);
    const int64_t o_eb = blob.add(enc_b.data(), enc_b.size() * 2);
    const int64_t o_ed = blob.add(desc.data(), desc.size() * 4);
    const int64_t o_gr = blob.add(grids.data(), grids.size() * 4);
    const int64_t o_da = blob.add(dec_a.data(), dec_a.size() * 2);
    const int64_t o_ds = blob.add(dscale.data(), dscale.size() * 4);
    const int64_t o_fd = blob.add(fields.data(), fields.size() * 4);
    const int64_t o_hl = blob.add(cb_hl.data(), cb_hl.size() * 2);
    const int64_t o_h = blob.add(cb_h.data(), cb_h.size() * 2);
    const int64_t o_u = blob.add(U32.data(), U32.size() * 4);
    const int64_t o_sg = blob.add(sig.data(), sig.size() * 4);

    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess) return TQ_EHIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return TQ_EHIP;
    void* mem = nullptr;
    if (hipMalloc(&mem, blob.host.size()) != hipSuccess) return TQ_EHIP;
    if (hipMemcpy(mem, blob.host.data(), blob.host.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(mem);
        return TQ_EHIP;
    }
    uint8_t* base = static_cast<uint8_t*>(mem);
    tq_sq_codec* c = new tq_sq_codec();
    SqDev& t = c->dev;
    t.d = d;
    t.n_heads = H;
    t.rec_words = rec_words;
    t.enc_b = reinterpret_cast<const _Float16*>(base + o_eb);
    t.enc_desc = reinterpret_cast<const float4*>(base + o_ed);
    t.grids = reinterpret_cast<const uint32_t*>(base + o_gr);
    t.lds_grid_words = (int)grids.size();
    t.dec_a = reinterpret_cast<const _Float16*>(base + o_da);
    t.dec_scale = reinterpret_cast<const float*>(base + o_ds);
    t.fields = reinterpret_cast<const uint4*>(base + o_fd);
    t.cb_hl = reinterpret_cast<const _Float16*>(base + o_hl);
    t.cb_h = reinterpret_cast<const _Float16*>(base + o_h);
    t.U32 = reinterpret_cast<const float*>(base + o_u);
    t.sigma = reinterpret_cast<const float*>(base + o_sg);
    t.m = M;
    t.sk_b = reinterpret_cast<const _Float16*>(base + o_skb);
    t.sk32 = reinterpret_cast<const float*>(base + o_sk32);
    t.sk_off = reinterpret_cast<const int32_t*>(base + o_skoff);
    t.deff = reinterpret_cast<const int32_t*>(base + o_deff);
    t.cent32 = reinterpret_cast<const float*>(base + o_c32);
    t.pm1 = reinterpret_cast<const _Float16*>(base + o_pm1);
    t.blob = mem;
    c->device = device;
    c->num_cus = cus;
    *out = c;
    return TQ_OK;
}

void tq_sq_destroy(tq_sq_codec* codec) {
    if (!codec) return;
    int cur = 0;
    const bool switched = hipGetDevice(&cur) == hipSuccess && cur != codec->device &&
                          hipSetDevice(codec->device) == hipSuccess;
    (void)hipFree(codec->dev.blob);
    if (switched) (void)hipSetDevice(cur);
    delete codec;
}

int tq_sq_record_bytes(const tq_sq_codec* codec, int64_t* bytes) {
    if (!codec || !bytes) return TQ_EINVAL;
    *bytes = (int64_t)codec->dev.rec_words * 4;
    return TQ_OK;
}

int tq_sq_encode(const tq_sq_codec* codec, const void* x, tq_dtype x_dtype, int64_t n_streams,
                 int64_t n_tokens, void* packed, void* stream) {
    if (!codec || n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    if (x_dtype != TQ_BF16) return x_dtype == TQ_F32 || x_dtype == TQ_F16 ? TQ_EUNSUPPORTED : TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0) return TQ_OK;
    if (!x || !packed) return TQ_EINVAL;
    if (!aligned16(x) || !aligned16(packed)) return TQ_EALIGN;
    if (!on_codec_device(codec)) return TQ_EINVAL;
    SqEncodeArgs a{};
    a.t = codec->dev;
    a.x = static_cast<const uint16_t*>(x);
    a.out = static_cast<uint32_t*>(packed);
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    return launch_sq_encode(a, codec->num_cus, static_cast<hipStream_t>(stream)) == hipSuccess ? TQ_OK : TQ_EHIP;
}

int tq_sq_decode(const tq_sq_codec* codec, const void* packed, int64_t n_streams, int64_t n_tokens,
                 void* x_hat, tq_dtype out_dtype, void* stream) {
    if (!codec || n_streams < 0 || n_tokens < 0) return TQ_EINVAL;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return out_dtype == TQ_F16 ? TQ_EUNSUPPORTED : TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0) return TQ_OK;
    if (!packed || !x_hat) return TQ_EINVAL;
    if (!aligned16(packed) || !aligned16(x_hat)) return TQ_EALIGN;
    if (!on_codec_device(codec)) return TQ_EINVAL;
    SqDecodeArgs a{};
    a.t = codec->dev;
    a.in = static_cast<const uint32_t*>(packed);
    a.out = x_hat;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    return launch_sq_decode(a, out_dtype == TQ_BF16, codec->num_cus, static_cast<hipStream_t>(stream)) == hipSuccess
               ? TQ_OK : TQ_EHIP;
}

namespace {
// scores workspace: projected queries (fp16), their scales, and with a sketch S q_Z (64 fp16 per row)
// and its scales
struct SqScoresWs {
    int64_t o_qs, o_pp, o_ps, o_ql, o_pl, total;
};
SqScoresWs sq_scores_ws(const tq_sq_codec* codec, int64_t n_streams, int64_t n_q) {
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t rows = n_streams * ((n_q + 15) / 16 * 16);
    const bool sk = codec->dev.m > 0;
    SqScoresWs w{};
    w.o_qs = al(rows * codec->dev.d * 2);
    w.o_pp = w.o_qs + al(rows * 4);
    w.o_ps = w.o_pp + (sk ? al(rows * 64 * 2) : 0);
    w.o_ql = w.o_ps + (sk ? al(rows * 4) : 0);
    w.o_pl = w.o_ql + al(rows * codec->dev.d * 2);
    w.total = w.o_pl + (sk ? al(rows * 64 * 2) : 0);
    return w;
}
}  // namespace

size_t tq_sq_scores_workspace_bytes(const tq_sq_codec* codec, int64_t n_streams, int64_t n_q) {
    if (!codec || n_streams < 0 || n_q < 0) return 0;
    return (size_t)sq_scores_ws(codec, n_streams, n_q).total;
}

int tq_sq_qk_scores(const tq_sq_codec* codec, const void* q, tq_dtype q_dtype, int64_t n_q,
                    const void* packed_k, int64_t n_streams, int64_t n_tokens, float* scores,
                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!codec || n_streams < 0 || n_tokens < 0 || n_q < 0 || n_q > 256) return TQ_EINVAL;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return q_dtype == TQ_F16 ? TQ_EUNSUPPORTED : TQ_EINVAL;
    if (n_streams == 0 || n_tokens == 0 || n_q == 0) return TQ_OK;
    if (!q || !packed_k || !scores || !workspace) return TQ_EINVAL;
    if (!aligned16(q) || !aligned16(packed_k) || !aligned16(scores) || !aligned16(workspace)) return TQ_EALIGN;
    if (workspace_bytes < tq_sq_scores_workspace_bytes(codec, n_streams, n_q)) return TQ_EWORKSPACE;
    if (!on_codec_device(codec)) return TQ_EINVAL;
    SqScoresArgs a{};
    a.t = codec->dev;
    a.q = q;
    a.q_bf16 = q_dtype == TQ_BF16;
    a.in = static_cast<const uint32_t*>(packed_k);
    a.scores = scores;
    a.n_streams = n_streams;
    a.n_tokens = n_tokens;
    a.n_q = n_q;
    a.nq_pad = (n_q + 15) / 16 * 16;
    const SqScoresWs w = sq_scores_ws(codec, n_streams, n_q);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.qp = reinterpret_cast<_Float16*>(ws);
    a.qscale = reinterpret_cast<float*>(ws + w.o_qs);
    a.qplo = reinterpret_cast<_Float16*>(ws + w.o_ql);
    if (codec->dev.m > 0) {
        a.pp = reinterpret_cast<_Float16*>(ws + w.o_pp);
        a.pscale = reinterpret_cast<float*>(ws + w.o_ps);
        a.pplo = reinterpret_cast<_Float16*>(ws + w.o_pl);
    }
    a.qmul = 1.0f;
    a.tiles_per_stream = (n_tokens + 15) / 16;
    return launch_sq_scores(a, codec->num_cus, static_cast<hipStream_t>(stream)) == hipSuccess ? TQ_OK : TQ_EHIP;
}

size_t tq_sq_attention_workspace_bytes(const tq_sq_codec* ck, int32_t batch, int32_t n_q_heads,
                                       int32_t n_kv_heads, int64_t n_tokens) {
    if (!ck || batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_tokens < 0) return 0;
    return (size_t)sq_attn_ws(ck->dev.d, ck->dev.m, (int64_t)batch * n_kv_heads, n_tokens).total;
}

int tq_sq_decode_attention(const tq_sq_codec* ck, const tq_sq_codec* cv, const void* q, tq_dtype q_dtype,
                           int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const void* packed_k,
                           const void* packed_v, int64_t n_tokens, const int32_t* lengths,
                           float softmax_scale, void* out, tq_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!ck || !cv || batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_tokens < 0) return TQ_EINVAL;
    if (n_q_heads % n_kv_heads != 0 || n_q_heads / n_kv_heads > 16) return TQ_EINVAL;
    if (ck->dev.d != cv->dev.d || ck->dev.n_heads != n_kv_heads || cv->dev.n_heads != n_kv_heads) return TQ_EINVAL;
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
    const SqAttnWs w = sq_attn_ws(ck->dev.d, ck->dev.m, streams, n_tokens);
    if (workspace_bytes < (size_t)w.total) return TQ_EWORKSPACE;
    if (!on_codec_device(ck) || !on_codec_device(cv)) return TQ_EINVAL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)ck->dev.d);
    SqScoresArgs qa{};
    qa.t = ck->dev;
    qa.q = q;
    qa.q_bf16 = q_dtype == TQ_BF16;
    qa.qp = reinterpret_cast<_Float16*>(ws);
    qa.qscale = reinterpret_cast<float*>(ws + w.o_qs);
    qa.qplo = reinterpret_cast<_Float16*>(ws + w.o_ql);
    if (ck->dev.m > 0) {
        qa.pp = reinterpret_cast<_Float16*>(ws + w.o_pp);
        qa.pscale = reinterpret_cast<float*>(ws + w.o_ps);
    }
    qa.qmul = scale * 1.4426950408889634f;   // scores in base-2 units for exp2
    qa.n_streams = streams;
    qa.n_q = n_q_heads / n_kv_heads;
    qa.nq_pad = 16;
    if (launch_sq_qprep(qa, s) != hipSuccess) return TQ_EHIP;
    SqAttnArgs a{};
    a.tk = ck->dev;
    a.tv = cv->dev;
    a.qp = qa.qp;
    a.qscale = qa.qscale;
    a.qplo = qa.qplo;
    a.pp = qa.pp;
    a.pscale = qa.pscale;
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
    return launch_sq_attention(a, s) == hipSuccess ? TQ_OK : TQ_EHIP;
}

int tq_sq_host_codebook(int32_t b, double* thresholds, double* centroids) {
    if (b < 1 || b > kBMax) return TQ_EINVAL;
    const GaussBook& g = gauss_book(b);
    if (thresholds) std::memcpy(thresholds, g.thr.data(), sizeof(double) * g.thr.size());
    if (centroids) std::memcpy(centroids, g.cent.data(), sizeof(double) * g.cent.size());
    return TQ_OK;
}

}  // extern "C"
