// tq4_codebook.cpp -- the 16 TQ4 centroids and 15 decision thresholds.
//
// The centroids are the 16-level minimum-mean-square-error (Lloyd-Max)
// quantiser of N(0,1), divided by 16 so that they quantise one coordinate of
// a rotated 256-dim unit vector (variance 1/256), rounded to fp32.  The
// thresholds are the fp32-rounded midpoints of adjacent fp32 centroids.
// ("centroid lookup" in "Fitting a 27B-Parameter LLM into 24 GiB of Laptop
// Memory", section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime";
// the pages give no values, so the level set is fixed by this construction.)
//
// Method: Max's shooting construction for a symmetric quantiser with an even
// number of levels.  The middle boundary is 0.  Given the smallest positive
// level y1, each cell's upper boundary follows from the centroid condition
// (solved by bisection) and the next level from the midpoint condition
// y_{j+1} = 2 x_j - y_j.  The outermost level must then equal the mean of the
// tail beyond the last boundary; y1 is found by bisection on that mismatch.
#include <cmath>
#include <mutex>

#include "tq4_launch.h"

namespace tq4 {
namespace {

double phi(double x) { return std::exp(-0.5 * x * x) * 0.39894228040143267794; }

// P(X > x) for X ~ N(0,1)
double tail(double x) { return 0.5 * std::erfc(x * 0.70710678118654752440); }

// E[X | a < X < b] for 0 <= a < b (b may be +inf)
double cond_mean(double a, double b) {
    const double mass = std::isinf(b) ? tail(a) : tail(a) - tail(b);
    const double mom = phi(a) - (std::isinf(b) ? 0.0 : phi(b));
    return mom / mass;
}

// March outward from y1. Returns +1 if y1 is too large (a centroid condition
// cannot be met or the last level overshoots its tail mean), -1 if too small.
// Fills the 8 positive levels and 7 positive boundaries on the way.
int march(double y1, double lev[8], double bnd[8]) {
    double lo_edge = 0.0;
    double y = y1;
    for (int j = 0; j < 7; ++j) {
        lev[j] = y;
        // need x with cond_mean(lo_edge, x) == y; cond_mean grows with x.
        if (cond_mean(lo_edge, INFINITY) <= y) return +1;
        if (y <= lo_edge) return -1;
        double a = lo_edge, b = lo_edge + 1.0;
        while (cond_mean(lo_edge, b) < y) b = lo_edge + 2.0 * (b - lo_edge);
        for (int it = 0; it < 200; ++it) {
            const double m = 0.5 * (a + b);
            if (m == a || m == b) break;
            if (cond_mean(lo_edge, m) < y) a = m; else b = m;
        }
        const double x = 0.5 * (a + b);
        bnd[j] = x;
        y = 2.0 * x - y;
        lo_edge = x;
        if (y <= x) return +1;
    }
    lev[7] = y;
    const double want = cond_mean(lo_edge, INFINITY);
    return y > want ? +1 : -1;
}

Codebook build() {
    double lev[8], bnd[8];
    double a = 1e-3, b = 1.0;  // bracket for the smallest positive level
    for (int it = 0; it < 200; ++it) {
        const double m = 0.5 * (a + b);
        if (m == a || m == b) break;
        if (march(m, lev, bnd) > 0) b = m; else a = m;
    }
    march(0.5 * (a + b), lev, bnd);
    Codebook cb;
    for (int i = 0; i < 8; ++i) {
        const float c = static_cast<float>(lev[i] / 16.0);
        cb.centroid[8 + i] = c;
        cb.centroid[7 - i] = -c;
    }
    for (int i = 0; i < 15; ++i)
        cb.threshold[i] = static_cast<float>(
            (static_cast<double>(cb.centroid[i]) + static_cast<double>(cb.centroid[i + 1])) * 0.5);
    return cb;
}

}  // namespace

const Codebook &codebook() {
    static std::once_flag once;
    static Codebook cb;
    std::call_once(once, [] { cb = build(); });
    return cb;
}

}  // namespace tq4
