// Host tables: SplitMix64 counters, Box-Muller Gaussians, and the Lloyd-Max codebook of the
// coordinate density of a random unit vector ("Ablation, Statistical Inference, and Validation for
// KV-Cache Compression", §2 TurboQuant: rotated coordinates ≈ Beta((d-1)/2,(d-1)/2) on [-1,1], one
// analytical Lloyd-Max codebook for all coordinates).
#include "tables.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>

namespace tq {

static constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t stream_key(uint64_t seed, uint32_t tag, uint32_t head) {
    return mix64(seed ^ mix64((uint64_t(tag) << 40) | uint64_t(head)));
}

void head_signs(uint64_t seed, uint32_t head, int d, std::vector<float>& out) {
    out.resize(d);
    uint64_t st = stream_key(seed, 1, head);
    for (int j = 0; j < d; ++j) {
        st += kGamma;
        out[j] = (mix64(st) >> 63) ? -1.0f : 1.0f;
    }
}

void rht_signs(uint64_t seed, uint32_t head, int d, std::vector<float>& out) {
    out.resize(d);
    uint64_t st = stream_key(seed, 3, head);
    for (int j = 0; j < d; ++j) {
        st += kGamma;
        out[j] = (mix64(st) >> 63) ? -1.0f : 1.0f;
    }
}

void rht_matrix_f16(uint64_t seed, uint32_t head, int d, std::vector<uint16_t>& out) {
    out.resize((size_t)d * d);
    std::vector<float> s2;
    rht_signs(seed, head, d, s2);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            const float v = ((__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0f : 1.0f) * s2[j];
            out[(size_t)i * d + j] = v > 0 ? 0x3c00u : 0xbc00u;   // fp16 +1 / -1
        }
}

uint16_t f64_to_f16_bits(double f) {
    _Float16 h = (_Float16)f;  // fptrunc double -> half: a single round-to-nearest-even
    uint16_t r;
    std::memcpy(&r, &h, 2);
    return r;
}

uint16_t f32_to_f16_bits(float f) { return f64_to_f16_bits((double)f); }  // exact widening first

float f16_bits_to_f32(uint16_t h) {
    _Float16 v;
    std::memcpy(&v, &h, 2);
    return (float)v;
}

void gaussian_matrix_f16(uint64_t seed, uint32_t head, int m, int d, std::vector<uint16_t>& out) {
    const int64_t n = int64_t(m) * d;
    out.resize(n);
    uint64_t st = stream_key(seed, 2, head);
    const double two_pi = 2.0 * M_PI;
    const double sc = std::ldexp(1.0, -53);
    for (int64_t e = 0; e < n; ++e) {
        st += kGamma;
        const uint64_t w0 = mix64(st);
        st += kGamma;
        const uint64_t w1 = mix64(st);
        const double u1 = double((w0 >> 11) + 1) * sc;  // (0, 1]
        const double u2 = double(w1 >> 11) * sc;        // [0, 1)
        out[e] = f64_to_f16_bits(std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2));
    }
}

// ---------------------------------------------------------------------------------------------
// Lloyd-Max.  With a = (d-1)/2 and alpha = a - 1, on a cell [lo, hi] of the positive half:
//   ∫ x (1-x^2)^alpha dx         = [(1-lo^2)^a - (1-hi^2)^a] / (2a)
//   ∫_y^1 (1-x^2)^alpha dx       = (1-y^2)^a · K(y) / (2a),  K(y) = CF((1-y)/2)
// where CF(x) is the continued fraction of the incomplete beta function with both parameters a,
//   I_x(a,a) = x^a (1-x)^a / (a B(a,a)) · CF(x),   CF(x) = 1/(1+ d1/(1+ d2/(1+ ...))),
//   d_{2k+1} = -(a+k)(2a+k) x / ((a+2k)(a+2k+1)),  d_{2k} = k (a-k) x / ((a+2k-1)(a+2k))
// (DLMF 8.17.22), evaluated by the modified Lentz method.  The centroid of a cell is then a ratio
// in which every normalising constant cancels.
// ---------------------------------------------------------------------------------------------
static double beta_cf(double a, double x) {
    const double tiny = 1e-300;
    // f = 1 / (1 + d1/(1 + d2/(1 + ...))): run Lentz on b0=1, a_k = d_k, b_k = 1 and invert.
    double f = 1.0, C = 1.0, D = 0.0;
    for (int n = 1; n < 100000; ++n) {
        double dn;
        if (n & 1) {
            const int k = (n - 1) / 2;
            dn = -(a + k) * (2.0 * a + k) * x / ((a + 2 * k) * (a + 2 * k + 1));
        } else {
            const int k = n / 2;
            dn = k * (a - k) * x / ((a + 2 * k - 1) * (a + 2 * k));
        }
        D = 1.0 + dn * D;
        if (std::fabs(D) < tiny) D = tiny;
        C = 1.0 + dn / C;
        if (std::fabs(C) < tiny) C = tiny;
        D = 1.0 / D;
        const double delta = C * D;
        f *= delta;
        if (std::fabs(delta - 1.0) < 1e-17) break;
    }
    return 1.0 / f;
}

static double pow_1my2(double y, double a) { return std::pow((1.0 - y) * (1.0 + y), a); }

// unnormalised upper-tail mass ×2a:  (1-y^2)^a · CF((1-y)/2), valid for 0 <= y <= 1
static double upper_tail(double y, double a) {
    if (y >= 1.0) return 0.0;
    return pow_1my2(y, a) * beta_cf(a, 0.5 * (1.0 - y));
}

int lloyd_max(int d, int b, std::vector<double>& thresholds, std::vector<double>& centroids) {
    if (d < 4 || b < 1 || b > 12) return -1;
    const int L = 1 << b, K = L / 2;
    const double a = 0.5 * (d - 1);
    std::vector<double> c(K), t(K + 1), tail(K + 1), pw(K + 1);
    // start: equal-mass positive cells of a Gaussian with the same variance 1/d (any interior start
    // converges: the density is log-concave, so the Lloyd fixed point is unique)
    for (int k = 0; k < K; ++k) {
        const double p = (K + k + 0.5) / L;  // target cdf
        // inverse normal cdf by bisection on erfc (host, start values only)
        double lo = -10, hi = 10;
        for (int it = 0; it < 200; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
        }
        c[k] = std::min(0.999, 0.5 * (lo + hi) / std::sqrt((double)d));
    }
    auto sweep = [&](std::vector<double>& cn) {
        t[0] = 0.0;
        t[K] = 1.0;
        for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        for (int k = 0; k <= K; ++k) {
            tail[k] = upper_tail(t[k], a);
            pw[k] = t[k] >= 1.0 ? 0.0 : pow_1my2(t[k], a);
        }
        double delta = 0.0;
        for (int k = 0; k < K; ++k) {
            cn[k] = (pw[k] - pw[k + 1]) / (tail[k] - tail[k + 1]);
            delta = std::max(delta, std::fabs(cn[k] - c[k]));
        }
        return delta;
    };
    std::vector<double> cn(K);
    // Lloyd sweeps until the transient has died out ...
    for (int it = 0; it < 200000; ++it) {
        const double delta = sweep(cn);
        c.swap(cn);
        if (delta < 1e-7 || K == 1) break;
    }
    // ... then Newton on R_k(c) = c_k·mass_k - moment_k = 0 with thresholds at the midpoints
    // (tridiagonal Jacobian; all integrals carry the same factor 2a).
    if (K > 1) {
        std::vector<double> fpdf(K + 1), mass(K), R(K), lo(K), di(K), up(K), cp(K), dp(K), dc(K);
        for (int it = 0; it < 100; ++it) {
            t[0] = 0.0;
            t[K] = 1.0;
            for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
            for (int k = 0; k <= K; ++k) {
                tail[k] = upper_tail(t[k], a);
                pw[k] = t[k] >= 1.0 ? 0.0 : pow_1my2(t[k], a);
                fpdf[k] = t[k] >= 1.0 ? 0.0 : 2.0 * a * std::pow((1.0 - t[k]) * (1.0 + t[k]), a - 1.0);
            }
            for (int k = 0; k < K; ++k) {
                mass[k] = tail[k] - tail[k + 1];
                R[k] = c[k] * mass[k] - (pw[k] - pw[k + 1]);
                const double dhi = (k + 1 < K) ? (c[k] - t[k + 1]) * fpdf[k + 1] : 0.0;
                const double dlo = (k > 0) ? (t[k] - c[k]) * fpdf[k] : 0.0;
                di[k] = mass[k] + 0.5 * dhi + 0.5 * dlo;
                up[k] = 0.5 * dhi;
                lo[k] = 0.5 * dlo;
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
    thresholds.assign(L - 1, 0.0);
    centroids.assign(L, 0.0);
    for (int k = 0; k < K; ++k) {
        centroids[K + k] = c[k];
        centroids[K - 1 - k] = -c[k];
    }
    for (int k = 0; k < L - 1; ++k) thresholds[k] = 0.5 * (centroids[k] + centroids[k + 1]);
    return 0;
}

// ---------------------------------------------------------------------------------------------
bool build_grid(const std::vector<double>& thr_y, Grid& out) {
    const double eps = 1.0 / 256.0;  // in u units; the fp32 rounding of u is below 2^-11
    for (int G = 64; G <= 4096; G *= 2) {
        const double gA = 0.5 * G, gB = 0.5 * G + 1.0;
        std::vector<float> tu(thr_y.size());
        for (size_t k = 0; k < thr_y.size(); ++k) tu[k] = (float)(thr_y[k] * gA + gB);
        std::vector<uint32_t> e(2 * (G + 3));
        bool ok = true;
        for (int c = 0; c < G + 3 && ok; ++c) {
            const double lo = c - eps, hi = c + 1 + eps;
            int base = 0, inside = 0;
            float cand = std::numeric_limits<float>::infinity();
            for (float tf : tu) {
                if ((double)tf < lo) ++base;
                else if ((double)tf <= hi) { ++inside; cand = tf; }
            }
            if (inside > 1) ok = false;
            if (c == 0) { base = 0; cand = std::numeric_limits<float>::infinity(); }
            uint32_t bits;
            std::memcpy(&bits, &cand, 4);
            e[2 * c] = bits;
            e[2 * c + 1] = (uint32_t)base;
        }
        if (ok) {
            out.G = G;
            out.thr_u.swap(tu);
            out.entries.swap(e);
            return true;
        }
    }
    return false;
}

bool build_fq_grid(const std::vector<double>& thr_y, int b, std::vector<uint32_t>& E) {
    if (b < 1 || b > 4) return false;
    std::vector<uint32_t> T(thr_y.size());
    for (size_t k = 0; k < thr_y.size(); ++k) {
        const float f = (float)(3.0 + kFqKappa * thr_y[k]);
        std::memcpy(&T[k], &f, 4);
        if (T[k] < 0x40000000u || T[k] >= 0x40800000u) return false;
    }
    E.assign(128, 0u);
    for (uint32_t c = 0; c < 128; ++c) {
        const uint32_t lo = 0x40000000u + (c << 16), hi = lo + 0x10000u;
        uint64_t base = 0;
        int inside = 0;
        uint32_t tc = hi;
        for (uint32_t t : T) {
            if (t < lo) ++base;
            else if (t < hi) { ++inside; tc = t; }
        }
        if (inside > 1) return false;
        E[c] = (uint32_t)(((base + 1) << (32 - b)) - (uint64_t)tc);
    }
    return true;
}

}  // namespace tq
