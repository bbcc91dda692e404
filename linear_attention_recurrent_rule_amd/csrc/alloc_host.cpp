// Lifetime-aware pivot and width assignment, run on the host once per
// calibration (STEPQuant paper, arXiv 2609.38169: App. A.3 "Mean log
// retention" for the lifetime weight; App. C.2 "KDA calibration" for the
// pivot ranking, "Allocation optimizers" and Table C1 for the per-unit
// Lagrangian with a shared multiplier followed by a repair).
//
// Units are the key rows of every value head.  Objective per unit and width
// b: L_u d_u(b), L_u = sum_{j<H} exp(2 j ell_u) the lifetime weight of the
// unit's mean log retention ell_u, d_u(b) its candidate distortion.
//
//  1. Pivots: the n_pivot units of largest L_u (d_u(b_nom) - d_u(FP16)); a
//     strict order (score, then lower unit first) makes the set unique.
//  2. Every other unit's useful widths are the vertices of the lower convex
//     hull of its points (b, L_u d_u(b)) up to the last one that still lowers
//     the objective.  Moving along the hull from width b to b' saves
//     (L d(b) - L d(b')) / (b' - b) per bit; along a convex hull these
//     savings decrease, so the Lagrangian minimiser of L d(b) + lambda b is
//     the vertex after the last step whose saving exceeds lambda.
//  3. The shared multiplier: every step of every unit is a breakpoint; the
//     steps are ordered by decreasing saving (ties: lower unit, then lower
//     width), and bisection over that order finds the longest prefix whose
//     per-unit minimisers fit the budget b_nom * (number of integer units).
//  4. Repair: the remaining steps are considered in the same order, one unit
//     at a time through a queue of each unit's next step; a step that fits is
//     taken, a unit whose next step does not fit keeps its width.
//
// The result is a function of the statistics alone.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <queue>
#include <vector>

#include "stq_internal.h"

namespace stq {

namespace {

constexpr int kWidth[kNumClasses] = {16, 8, 6, 4, 2};

// Lifetime weight: the geometric series 1 + e^{2l} + ... + e^{2(H-1)l} in
// closed form, (e^{2Hl} - 1) / (e^{2l} - 1), accurate through expm1 when the
// retention is close to one; H when the retention is exactly one.
double lifetime_weight(double ell, int horizon) {
    if (ell == 0.0) return static_cast<double>(horizon);
    return std::expm1(2.0 * horizon * ell) / std::expm1(2.0 * ell);
}

// A breakpoint: the step of unit u from hull vertex s to s + 1.
struct Breakpoint {
    double saving; // objective saved per bit
    int unit;
    int s;
    int bits;      // width added by the step
};

// Order of the breakpoints (and of the multiplier): larger saving first; on
// equal savings the lower unit, then the lower width, goes first.
bool before(const Breakpoint &x, const Breakpoint &y) {
    if (x.saving != y.saving) return x.saving > y.saving;
    if (x.unit != y.unit) return x.unit < y.unit;
    return x.s < y.s;
}

// Lower hull of one unit's candidate points by gift wrapping: from the
// current vertex go to the later candidate with the largest saving per bit
// (on a tie the farthest one, so collinear middle points are skipped); stop
// when no later candidate lowers the objective.  cost[k], width[k] for the
// candidates in increasing width; returns the vertex indices.
void hull_of(const std::vector<double> &cost, const std::vector<int> &width, std::vector<int> &hull) {
    hull.clear();
    const int n = static_cast<int>(cost.size());
    int v = 0;
    hull.push_back(v);
    while (v + 1 < n) {
        int best = -1;
        double best_saving = 0.0;
        for (int k = v + 1; k < n; ++k) {
            const double saving = (cost[v] - cost[k]) / static_cast<double>(width[k] - width[v]);
            if (best < 0 || saving >= best_saving) { // ties go to the farther point
                best = k;
                best_saving = saving;
            }
        }
        if (!(best_saving > 0.0)) break;
        hull.push_back(best);
        v = best;
    }
}

} // namespace

bool assign_rows(int Hv, int D, const double *dist, const double *logret, double n,
                 int horizon, unsigned cand_mask, int nominal, int n_pivot, int32_t *counts,
                 int32_t *perm) {
    const int N = Hv * D;
    if (!(n > 0.0) || horizon < 1 || n_pivot < 0 || n_pivot > N) return false;
    // integer candidate classes, in increasing width
    std::vector<int> cls;
    for (int k = kNumClasses - 1; k >= 1; --k)
        if (cand_mask & (1u << k)) cls.push_back(k);
    int k_nom = -1;
    for (int k : cls)
        if (kWidth[k] == nominal) k_nom = k;
    if (cls.empty() || k_nom < 0) return false;
    auto d = [&](int u, int k) { return dist[static_cast<size_t>(u) * kNumClasses + k]; };

    std::vector<double> L(N);
    for (int u = 0; u < N; ++u) L[u] = lifetime_weight(logret[u] / n, horizon);

    // ---- 1. pivots: the n_pivot first units in the strict order of their
    // lifetime-weighted distortion reduction from b_nom to FP16
    std::vector<char> pivot(N, 0);
    if (n_pivot > 0) {
        std::vector<int> ids(N);
        for (int u = 0; u < N; ++u) ids[u] = u;
        auto more_risk = [&](int x, int y) {
            const double sx = L[x] * (d(x, k_nom) - d(x, 0)), sy = L[y] * (d(y, k_nom) - d(y, 0));
            return sx != sy ? sx > sy : x < y;
        };
        std::nth_element(ids.begin(), ids.begin() + (n_pivot - 1), ids.end(), more_risk);
        for (int r = 0; r < n_pivot; ++r) pivot[ids[r]] = 1;
    }

    // ---- 2. per-unit hulls and their steps
    const int nc = static_cast<int>(cls.size());
    std::vector<std::vector<int>> hulls(N);
    std::vector<std::vector<Breakpoint>> steps(N);
    std::vector<Breakpoint> bps;
    std::vector<double> cost(nc);
    std::vector<int> width(nc);
    for (int k = 0; k < nc; ++k) width[k] = kWidth[cls[k]];
    long long n_int = 0;
    for (int u = 0; u < N; ++u) {
        if (pivot[u]) continue;
        ++n_int;
        for (int k = 0; k < nc; ++k) cost[k] = L[u] * d(u, cls[k]);
        hull_of(cost, width, hulls[u]);
        const std::vector<int> &hu = hulls[u];
        for (int s = 0; s + 1 < static_cast<int>(hu.size()); ++s) {
            const int db = width[hu[s + 1]] - width[hu[s]];
            steps[u].push_back({(cost[hu[s]] - cost[hu[s + 1]]) / static_cast<double>(db), u, s, db});
        }
        bps.insert(bps.end(), steps[u].begin(), steps[u].end());
    }
    const long long budget = static_cast<long long>(nominal) * n_int;
    const long long base = static_cast<long long>(width[0]) * n_int;
    if (base > budget) return false;

    // ---- 3. the shared multiplier.  At position m of the order (m == S: below
    // every breakpoint) each unit's Lagrangian minimiser takes those of its
    // steps that come before position m; the total width grows with m, and
    // bisection finds the last position whose minimisers fit the budget.
    std::sort(bps.begin(), bps.end(), before);
    const int S = static_cast<int>(bps.size());
    auto minimisers = [&](int m, std::vector<int> &lev) -> long long {
        long long total = base;
        for (int u = 0; u < N; ++u) {
            int s = 0;
            for (const Breakpoint &b : steps[u]) {
                if (m < S && !before(b, bps[m])) break;
                total += b.bits;
                ++s;
            }
            lev[u] = s;
        }
        return total;
    };
    std::vector<int> level(N, 0);
    int lo = 0; // the minimisers at lo fit (at 0 every unit has its narrowest width)
    if (minimisers(S, level) <= budget) {
        lo = S;
    } else {
        int hi = S; // the minimisers at hi do not fit
        while (hi - lo > 1) {
            const int mid = lo + (hi - lo) / 2;
            if (minimisers(mid, level) <= budget) lo = mid;
            else hi = mid;
        }
    }
    long long used = minimisers(lo, level);

    // ---- 4. repair: one queue entry per unit with a step left, holding that
    // unit's next step; the entry first in the order is decided next (the
    // first of all is the breakpoint at lo, which does not fit).
    auto later = [](const Breakpoint &x, const Breakpoint &y) { return before(y, x); };
    std::priority_queue<Breakpoint, std::vector<Breakpoint>, decltype(later)> next(later);
    for (int u = 0; u < N; ++u)
        if (level[u] < static_cast<int>(steps[u].size())) next.push(steps[u][level[u]]);
    while (!next.empty()) {
        const Breakpoint b = next.top();
        next.pop();
        if (used + b.bits > budget) continue; // the unit keeps its width
        used += b.bits;
        level[b.unit] = b.s + 1;
        if (b.s + 1 < static_cast<int>(steps[b.unit].size())) next.push(steps[b.unit][b.s + 1]);
    }

    // ---- class per row; per head the rows grouped by class (pivots, then
    // 8, 6, 4, 2 bits), each group in increasing logical row
    for (int h = 0; h < Hv; ++h) {
        std::vector<int> rows(D), klass(D);
        for (int i = 0; i < D; ++i) {
            const int u = h * D + i;
            rows[i] = i;
            klass[i] = pivot[u] ? 0 : cls[hulls[u][level[u]]];
        }
        std::stable_sort(rows.begin(), rows.end(), [&](int x, int y) { return klass[x] < klass[y]; });
        for (int k = 0; k < kNumClasses; ++k) counts[h * kNumClasses + k] = 0;
        for (int p = 0; p < D; ++p) {
            perm[h * D + p] = rows[p];
            ++counts[h * kNumClasses + klass[rows[p]]];
        }
    }
    return true;
}

} // namespace stq
