// Level tables and the exact nearest-level lookup of the quantize kernel (host code).
//
// NF4: "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 QLoRA / NF4, 【原理】①: the
// N(0,1) CDF is cut into 16 slabs of equal probability and each level is the
// representative midpoint of its slab, normalised to [-1, 1].  The midpoint is
// taken in probability, (2i+1)/32, and the quantiles are divided by the largest.
// FP4: same page, 【代码】: a generic float-format table with 2 exponent bits,
// 1 mantissa bit and a sign, 4 bits in all (IEEE-style, with subnormals).
#include <cmath>
#include <cstring>
#include <vector>
#include <algorithm>

#include "qk_internal.h"

namespace qk {

// Wichura, M. J. (1988) "Algorithm AS 241: The percentage points of the normal
// distribution", Applied Statistics 37(3), 477-484 — PPND16, about 16 digits.
double normal_quantile(double p) {
    static const double a[8] = {3.3871328727963666080e0, 1.3314166789178437745e+2,
                                1.9715909503065514427e+3, 1.3731693765509461125e+4,
                                4.5921953931549871457e+4, 6.7265770927008700853e+4,
                                3.3430575583588128105e+4, 2.5090809287301226727e+3};
    static const double b[8] = {1.0, 4.2313330701600911252e+1, 6.8718700749205790830e+2,
                                5.3941960214247511077e+3, 2.1213794301586595867e+4,
                                3.9307895800092710610e+4, 2.8729085735721942674e+4,
                                5.2264952788528545610e+3};
    static const double c[8] = {1.42343711074968357734e0, 4.63033784615654529590e0,
                                5.76949722146069140550e0, 3.64784832476320460504e0,
                                1.27045825245236838258e0, 2.41780725177450611770e-1,
                                2.27238449892691845833e-2, 7.74545014278341407640e-4};
    static const double d[8] = {1.0, 2.05319162663775882187e0, 1.67638483018380384940e0,
                                6.89767334985100004550e-1, 1.48103976427480074590e-1,
                                1.51986665636164571966e-2, 5.47593808499534494600e-4,
                                1.05075007164441684324e-9};
    static const double e[8] = {6.65790464350110377720e0, 5.46378491116411436990e0,
                                1.78482653991729133580e0, 2.96560571828504891230e-1,
                                2.65321895265761230930e-2, 1.24266094738807843860e-3,
                                2.71155556874348757815e-5, 2.01033439929228813265e-7};
    static const double f[8] = {1.0, 5.99832206555887937690e-1, 1.36929880922735805310e-1,
                                1.48753612908506148525e-2, 7.86869131145613259100e-4,
                                1.84631831751005468180e-5, 1.42151175831644588870e-7,
                                2.04426310338993978564e-15};
    auto poly = [](const double* k, double x) {
        double acc = k[7];
        for (int i = 6; i >= 0; --i) acc = acc * x + k[i];
        return acc;
    };
    const double q = p - 0.5;
    if (std::fabs(q) <= 0.425) {
        const double r = 0.180625 - q * q;
        return q * poly(a, r) / poly(b, r);
    }
    double r = q < 0 ? p : 1.0 - p;
    r = std::sqrt(-std::log(r));
    double v;
    if (r <= 5.0) {
        r -= 1.6;
        v = poly(c, r) / poly(d, r);
    } else {
        r -= 5.0;
        v = poly(e, r) / poly(f, r);
    }
    return q < 0 ? -v : v;
}

qk_status make_nf4(float out[16]) {
    double qv[16];
    for (int i = 0; i < 16; ++i) qv[i] = normal_quantile((2.0 * i + 1.0) / 32.0);
    for (int i = 0; i < 16; ++i) out[i] = (float)(qv[i] / qv[15]);
    out[0] = -1.0f;   // q_0 / q_15 is exactly -1 by symmetry of the quantile
    out[15] = 1.0f;
    return QK_OK;
}

qk_status make_fp4(float out[16]) {
    // code = s<<3 | e<<1 | m, bias 1: e == 0 -> m/2 * 2^0 (subnormal), else (1 + m/2) * 2^(e-1)
    for (int code = 0; code < 16; ++code) {
        const int s = (code >> 3) & 1, ex = (code >> 1) & 3, m = code & 1;
        const float mag = ex == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * std::ldexp(1.0f, ex - 1);
        const float v = mag / 6.0f;   // largest magnitude is 6 (e = 3, m = 1)
        out[code] = s ? -v : v;
    }
    return QK_OK;
}

qk_status make_dynamic_map(int32_t is_signed, float out[256]) {
    // "篇2-bitsandbytes-具体观-算法与实现剖析", §2.3 8-bit Optimizers, 【原理】: 256
    // non-uniform levels shaped by the distribution, dense at zero, sparse in the
    // tails, maximising the code entropy.  Equal probability mass per level:
    // signed   q_i = Phi^-1((2i + 1) / 512)
    // unsigned q_i = Phi^-1(1/2 + (2i + 1) / 1024)   (the half-normal)
    double q[256];
    for (int i = 0; i < 256; ++i)
        q[i] = is_signed ? normal_quantile((2.0 * i + 1.0) / 512.0) : normal_quantile(0.5 + (2.0 * i + 1.0) / 1024.0);
    for (int i = 0; i < 256; ++i) out[i] = (float)(q[i] / q[255]);
    if (is_signed) out[0] = -1.0f;   // q_0 = -q_255 by symmetry of the quantile
    out[255] = 1.0f;
    return QK_OK;
}

namespace {

// bin index computed exactly as the kernel does: low 24 bits of fmaf(t, S, S + 2^23)
inline uint32_t bin_of(float t, float S, float C) {
    const float f = std::fmaf(t, S, C);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u & 0xFFFFFFu;
}

inline float next_up(float v) { return std::nextafterf(v, INFINITY); }
inline float next_down(float v) { return std::nextafterf(v, -INFINITY); }

}  // namespace

qk_status build_quant_lut(const float levels[16], QuantLut* lut, const char** why) {
    for (int i = 0; i < 16; ++i) {
        if (!std::isfinite(levels[i]) || levels[i] < -1.0f || levels[i] > 1.0f) {
            *why = "levels must be finite and within [-1, 1]";
            return QK_ERR_INVALID_ARG;
        }
    }
    // distinct values in increasing order, each with the smallest code carrying it
    std::vector<float> u;
    for (int i = 0; i < 16; ++i) {
        bool seen = false;
        for (float v : u) seen = seen || (v == levels[i]);   // +0 == -0
        if (!seen) u.push_back(levels[i]);
    }
    std::sort(u.begin(), u.end());
    const int U = (int)u.size();
    std::vector<int> code_of(U);
    for (int s = 0; s < U; ++s) {
        int best = 16;
        for (int i = 0; i < 16; ++i)
            if (levels[i] == u[s]) best = std::min(best, i);
        code_of[s] = best;
    }
    bool sorted = true;
    for (int s = 0; s < U; ++s) sorted = sorted && (code_of[s] == s);
    sorted = sorted && U == 16;

    // threshold between u[s] and u[s+1]: the least binary32 t that maps to u[s+1]
    std::vector<float> T(U > 1 ? U - 1 : 0);
    for (int s = 0; s + 1 < U; ++s) {
        const double a = u[s], b = u[s + 1];
        const double m = (a + b) * 0.5;
        // exactness of the binary64 midpoint: (a + b) must not have rounded
        const double sum = a + b;
        const double bb = sum - a;
        if (bb != b || (sum - bb) != a) {
            *why = "a level midpoint is not exact in binary64";
            return QK_ERR_UNSUPPORTED;
        }
        const bool tie_goes_up = code_of[s + 1] < code_of[s];
        float t = (float)m;
        if (tie_goes_up) {
            while ((double)t < m) t = next_up(t);
            while ((double)next_down(t) >= m) t = next_down(t);
        } else {
            while ((double)t <= m) t = next_up(t);
            while ((double)next_down(t) > m) t = next_down(t);
        }
        T[s] = t;
    }

    for (int S = 8; S <= kLutMaxS; S *= 2) {
        const float Sf = (float)S, Cf = (float)S + 8388608.0f;
        const int nb = 2 * S + 1;
        std::vector<int> start_idx(nb, 0), inside_cnt(nb, 0), inside_thr(nb, -1);
        // sorted index at the lowest t of each bin, and thresholds falling inside bins
        std::vector<int> boundary_at(nb + 1, 0);
        for (int s = 0; s + 1 < U; ++s) {
            const uint32_t bt = bin_of(T[s], Sf, Cf);
            const uint32_t bp = bin_of(next_down(T[s]), Sf, Cf);
            if (bp == bt) {
                inside_cnt[bt] += 1;
                inside_thr[bt] = s;
            } else {
                boundary_at[bt] += 1;   // the step coincides with the start of bin bt
            }
        }
        bool ok = true;
        int cur = 0;
        for (int bi = 0; bi < nb; ++bi) {
            cur += boundary_at[bi];
            if (inside_cnt[bi] > 1) ok = false;
            start_idx[bi] = cur;
            cur += inside_cnt[bi];
        }
        if (!ok) continue;
        lut->S = Sf;
        lut->C = Cf;
        lut->nbins = nb;
        lut->sorted = sorted ? 1 : 0;
        lut->tiny_free = 1;
        for (int s = 0; s + 1 < U; ++s)
            if (T[s] > -0x1p-60f && T[s] <= 0x1p-60f) lut->tiny_free = 0;
        for (int bi = 0; bi < kLutMaxBins; ++bi) {
            lut->T[bi] = 2.0f;
            lut->c[bi] = 0;
        }
        for (int bi = 0; bi < nb; ++bi) {
            const int lo = start_idx[bi];
            const int clo = code_of[std::min(lo, U - 1)];
            // sorted tables: the kernel adds [t >= T] to c, so c holds the lower code only;
            // otherwise it selects bits 0..3 or 16..19 of c
            if (inside_cnt[bi] == 1) {
                const int chi = code_of[std::min(lo + 1, U - 1)];
                lut->T[bi] = T[inside_thr[bi]];
                lut->c[bi] = sorted ? (uint32_t)clo : ((uint32_t)clo | ((uint32_t)chi << 16));
            } else {
                lut->c[bi] = sorted ? (uint32_t)clo : ((uint32_t)clo | ((uint32_t)clo << 16));
            }
        }
        return QK_OK;
    }
    *why = "level thresholds are too close together for the lookup table";
    return QK_ERR_UNSUPPORTED;
}

namespace {

// Distinct values of a level table in increasing order, the smallest code carrying
// each, and the binary32 decision threshold between neighbours (the least t that
// maps to the upper value, the tie rule "smaller code wins" included).
qk_status sorted_thresholds(const float* levels, int nlev, std::vector<float>& u, std::vector<int>& code_of,
                            std::vector<float>& T, const char** why) {
    for (int i = 0; i < nlev; ++i) {
        if (!std::isfinite(levels[i]) || levels[i] < -1.0f || levels[i] > 1.0f) {
            *why = "levels must be finite and within [-1, 1]";
            return QK_ERR_INVALID_ARG;
        }
    }
    u.clear();
    for (int i = 0; i < nlev; ++i) u.push_back(levels[i]);
    std::sort(u.begin(), u.end());
    u.erase(std::unique(u.begin(), u.end(), [](float a, float b) { return a == b; }), u.end());   // +0 == -0
    const int U = (int)u.size();
    code_of.assign(U, nlev);
    for (int s = 0; s < U; ++s)
        for (int i = 0; i < nlev; ++i)
            if (levels[i] == u[s]) code_of[s] = std::min(code_of[s], i);
    T.assign(U > 1 ? U - 1 : 0, 0.0f);
    for (int s = 0; s + 1 < U; ++s) {
        const double a = u[s], b = u[s + 1];
        const double sum = a + b, bb = sum - a;
        if (bb != b || (sum - bb) != a) {
            *why = "a level midpoint is not exact in binary64";
            return QK_ERR_UNSUPPORTED;
        }
        const double m = sum * 0.5;
        const bool tie_goes_up = code_of[s + 1] < code_of[s];
        float t = (float)m;
        if (tie_goes_up) {
            while ((double)t < m) t = next_up(t);
            while ((double)next_down(t) >= m) t = next_down(t);
        } else {
            while ((double)t <= m) t = next_up(t);
            while ((double)next_down(t) > m) t = next_down(t);
        }
        T[s] = t;
    }
    return QK_OK;
}

}  // namespace

qk_status build_quant_lut8(const float levels[256], QuantLut8* lut, const char** why) {
    std::vector<float> u, T;
    std::vector<int> code_of;
    const qk_status st = sorted_thresholds(levels, 256, u, code_of, T, why);
    if (st != QK_OK) return st;
    const int U = (int)u.size();
    for (int S = 8; S <= kLut8MaxS; S *= 2) {
        const float Sf = (float)S, Cf = (float)S + 8388608.0f;
        // a threshold inside a bin (not at its first value) must be the only one there
        bool ok = true;
        uint32_t last_inside_bin = 0xFFFFFFFFu;
        for (int s = 0; s + 1 < U && ok; ++s) {
            const uint32_t bt = bin_of(T[s], Sf, Cf);
            if (bin_of(next_down(T[s]), Sf, Cf) == bt) {
                if (bt == last_inside_bin) ok = false;
                last_inside_bin = bt;
            }
        }
        if (!ok) continue;
        lut->S = Sf;
        lut->C = Cf;
        lut->nbins = 2 * S + 1;
        lut->nthr = U - 1;
        for (int s = 0; s < 255; ++s) lut->T[s] = s < U - 1 ? T[s] : 2.0f;
        for (int s = 0; s < 256; ++s) lut->code_of[s] = (uint8_t)code_of[std::min(s, U - 1)];
        return QK_OK;
    }
    *why = "level thresholds are too close together for the lookup table";
    return QK_ERR_UNSUPPORTED;
}

}  // namespace qk
