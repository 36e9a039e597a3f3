// The tachometer's fit (BASTION, "Methodik" §3, latency modelling: the
// verification latency follows a roofline model -- memory bandwidth, then
// compute -- calibrated on observed runtimes).  Host code: measured
// (N, time) pairs of a tree of N draft nodes are fitted by least squares to
//   C(N) = a + b N + c max(0, N - knee),
// the knee being where verification turns compute-bound.  Every integer knee
// of the range is tried; the three coefficients come from the normal
// equations (Gaussian elimination with partial pivoting, float64) and the
// knee with the smallest residual sum of squares wins (equal sums: the
// smaller knee).  A knee at or past every measured N fits c = 0.

#include <cmath>

#include "td_internal.h"

namespace {

// Solve the k x k system A x = y (k <= 3) in place; false if singular.
bool solve(int k, double (&A)[3][3], double (&y)[3], double (&x)[3]) {
    for (int col = 0; col < k; ++col) {
        int piv = col;
        for (int r = col + 1; r < k; ++r)
            if (std::fabs(A[r][col]) > std::fabs(A[piv][col])) piv = r;
        if (A[piv][col] == 0.0) return false;
        for (int j = 0; j < k; ++j) std::swap(A[col][j], A[piv][j]);
        std::swap(y[col], y[piv]);
        for (int r = col + 1; r < k; ++r) {
            const double f = A[r][col] / A[col][col];
            for (int j = col; j < k; ++j) A[r][j] -= f * A[col][j];
            y[r] -= f * y[col];
        }
    }
    for (int r = k - 1; r >= 0; --r) {
        double s = y[r];
        for (int j = r + 1; j < k; ++j) s -= A[r][j] * x[j];
        x[r] = s / A[r][r];
    }
    return true;
}

}  // namespace

using namespace td;

extern "C" td_status td_fit_cost(const double *n, const double *t, int32_t count, int32_t knee_min,
                                 int32_t knee_max, double *a, double *b, double *c, int32_t *knee,
                                 double *rss) {
    clear_error();
    if (!n || !t || !a || !b || !c || !knee) return fail(TD_EINVAL, "td_fit_cost: null pointer");
    if (count < 3) return fail(TD_EINVAL, "td_fit_cost: at least 3 measurements are needed");
    if (knee_min > knee_max) return fail(TD_EINVAL, "td_fit_cost: knee_min > knee_max");
    bool found = false;
    double best_rss = 0.0, best[3] = {0, 0, 0};
    int best_knee = knee_min;
    for (int kn = knee_min; kn <= knee_max; ++kn) {
        bool hinge_seen = false;
        for (int i = 0; i < count; ++i) hinge_seen = hinge_seen || n[i] > kn;
        const int k = hinge_seen ? 3 : 2;
        double A[3][3] = {}, y[3] = {}, x[3] = {0, 0, 0};
        for (int i = 0; i < count; ++i) {
            const double f[3] = {1.0, n[i], n[i] > kn ? n[i] - kn : 0.0};
            for (int r = 0; r < k; ++r) {
                for (int j = 0; j < k; ++j) A[r][j] += f[r] * f[j];
                y[r] += f[r] * t[i];
            }
        }
        if (!solve(k, A, y, x)) continue;
        double s = 0.0;
        for (int i = 0; i < count; ++i) {
            const double e = x[0] + x[1] * n[i] + x[2] * (n[i] > kn ? n[i] - kn : 0.0) - t[i];
            s += e * e;
        }
        if (!found || s < best_rss * (1.0 - 1e-12)) {
            found = true;
            best_rss = s;
            best[0] = x[0];
            best[1] = x[1];
            best[2] = x[2];
            best_knee = kn;
        }
    }
    if (!found) return fail(TD_EINVAL, "td_fit_cost: the measurements do not determine a line");
    *a = best[0];
    *b = best[1];
    *c = best[2];
    *knee = best_knee;
    if (rss) *rss = best_rss;
    return TD_OK;
}
