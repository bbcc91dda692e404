// Lifetime-aware pivot and width assignment, run on the host once per
// calibration (STEPQuant paper, arXiv 2609.38169: App. A.3 for the lifetime
// weight L_u = sum_{j<H} exp(2 j ell_u) with ell_u the mean log retention;
// App. C.2 "KDA calibration" for the pivot ranking and "Allocation
// optimizers" for the Lagrangian assignment with a repair step).
//
// Units are the key rows of every value head.  Pivots: the n_pivot units of
// largest L_u (d_u(b_nom) - d_u(FP16)).  Every other unit takes one of the
// candidate integer widths: on the lower convex hull of its points
// (b, L_u d_u(b)), hull steps are taken across all units in order of
// decreasing distortion saved per bit while the integer budget
// b_nom * (number of non-pivot units) holds, which follows the Lagrangian
// solutions of a shared multiplier; a unit whose next step no longer fits
// stops there and later steps of other units that still fit are taken (the
// repair).  Ties break by unit index, so the result is a pure function of
// the statistics.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "stq_internal.h"

namespace stq {

namespace {

constexpr int kWidth[kNumClasses] = {16, 8, 6, 4, 2};

struct Step {
    double gain; // distortion saved per bit
    int unit;
    int at;      // hull position the step starts from
};

} // namespace

bool assign_rows(int Hv, int D, const double *dist, const double *logret, double n,
                 int horizon, unsigned cand_mask, int nominal, int n_pivot, int32_t *counts,
                 int32_t *perm) {
    const int N = Hv * D;
    if (n <= 0.0 || horizon < 1 || n_pivot < 0 || n_pivot > N) return false;
    // candidate integer classes in ascending width
    std::vector<int> cand;
    int knom = -1;
    for (int k = kNumClasses - 1; k >= 1; --k)
        if (cand_mask & (1u << k)) {
            cand.push_back(k);
            if (kWidth[k] == nominal) knom = k;
        }
    if (cand.empty() || knom < 0) return false;

    // lifetime weights
    std::vector<double> L(N);
    for (int u = 0; u < N; ++u) {
        const double ell = logret[u] / n;
        double acc = 1.0;
        for (int j = 1; j < horizon; ++j) acc += std::exp(2.0 * static_cast<double>(j) * ell);
        L[u] = acc;
    }
    auto cost = [&](int u, int k) { return L[u] * dist[static_cast<size_t>(u) * kNumClasses + k]; };

    // pivots
    std::vector<int> order(N);
    for (int u = 0; u < N; ++u) order[u] = u;
    std::vector<double> score(N);
    for (int u = 0; u < N; ++u)
        score[u] = L[u] * (dist[static_cast<size_t>(u) * kNumClasses + knom] -
                           dist[static_cast<size_t>(u) * kNumClasses + 0]);
    std::sort(order.begin(), order.end(), [&](int x, int y) {
        if (score[x] != score[y]) return score[x] > score[y];
        return x < y;
    });
    std::vector<char> pivot(N, 0);
    for (int t = 0; t < n_pivot; ++t) pivot[order[t]] = 1;

    // hulls and steps
    const int nc = static_cast<int>(cand.size());
    std::vector<int> hull(static_cast<size_t>(N) * nc), hlen(N, 0), level(N, 0);
    std::vector<char> stopped(N, 0);
    std::vector<Step> steps;
    long n_int = 0;
    for (int u = 0; u < N; ++u) {
        if (pivot[u]) continue;
        ++n_int;
        int *hu = &hull[static_cast<size_t>(u) * nc];
        int m = 0;
        for (int a = 0; a < nc; ++a) {
            const double bx = kWidth[cand[a]], by = cost(u, cand[a]);
            while (m >= 2) {
                const double ox = kWidth[cand[hu[m - 2]]], oy = cost(u, cand[hu[m - 2]]);
                const double ax = kWidth[cand[hu[m - 1]]], ay = cost(u, cand[hu[m - 1]]);
                // drop the middle point unless it lies strictly below o-b
                if ((ax - ox) * (by - oy) - (ay - oy) * (bx - ox) <= 0.0)
                    --m;
                else
                    break;
            }
            hu[m++] = a;
        }
        int keep = 1;
        while (keep < m && cost(u, cand[hu[keep]]) < cost(u, cand[hu[keep - 1]])) ++keep;
        hlen[u] = keep;
        for (int s = 0; s + 1 < keep; ++s) {
            const double y0 = cost(u, cand[hu[s]]), y1 = cost(u, cand[hu[s + 1]]);
            const double db = static_cast<double>(kWidth[cand[hu[s + 1]]] - kWidth[cand[hu[s]]]);
            steps.push_back(Step{(y0 - y1) / db, u, s});
        }
    }
    const long budget = static_cast<long>(nominal) * n_int;
    long used = static_cast<long>(kWidth[cand[0]]) * n_int;
    if (used > budget) return false;
    std::sort(steps.begin(), steps.end(), [](const Step &x, const Step &y) {
        if (x.gain != y.gain) return x.gain > y.gain;
        if (x.unit != y.unit) return x.unit < y.unit;
        return x.at < y.at;
    });
    for (const Step &s : steps) {
        const int u = s.unit;
        if (stopped[u] || level[u] != s.at) continue;
        const int *hu = &hull[static_cast<size_t>(u) * nc];
        const long db = kWidth[cand[hu[s.at + 1]]] - kWidth[cand[hu[s.at]]];
        if (used + db <= budget) {
            used += db;
            level[u] = s.at + 1;
        } else {
            stopped[u] = 1;
        }
    }

    // class counts and physical order: pivots, 8, 6, 4, 2 bits, each class
    // in ascending logical row
    std::vector<int> cls(N);
    for (int u = 0; u < N; ++u)
        cls[u] = pivot[u] ? 0 : cand[hull[static_cast<size_t>(u) * nc + level[u]]];
    for (int h = 0; h < Hv; ++h) {
        for (int k = 0; k < kNumClasses; ++k) counts[h * kNumClasses + k] = 0;
        int p = 0;
        for (int k = 0; k < kNumClasses; ++k)
            for (int i = 0; i < D; ++i)
                if (cls[h * D + i] == k) {
                    perm[h * D + p++] = i;
                    ++counts[h * kNumClasses + k];
                }
    }
    return true;
}

} // namespace stq
