"""The library's lifetime-aware assignment (stq_assign_rows: pivots and row
widths, STEPQuant paper App. C.2 "KDA calibration" and "Allocation
optimizers", Table C1; lifetime weights App. A.3 "Mean log retention")
against the oracle's, bit for bit: identical class counts and row orders on
seeded instances chosen to reach every decision of the procedure - exact ties
of pivot scores and of hull slopes inside a head and across heads, collinear
and non-decreasing candidate points, budgets where the repair has to skip a
step that does not fit and take later ones, pivot counts from none to every
row, both candidate sets of Table C1 and others.  Host code only: no GPU.

The two implementations share nothing: the library builds each row's hull by
gift wrapping, finds the multiplier by bisection over the sorted hull slopes
and repairs through a queue of each row's next step, with the lifetime weight
in closed form; the oracle builds hulls by a monotone chain, sums the
weight's series term by term and walks the sorted slopes once."""
from __future__ import annotations

import numpy as np
import pytest

stq = pytest.importorskip("linear_attention_recurrent_rule_amd.stq")

CLASS = {8: 1, 6: 2, 4: 3, 2: 4}


def _mask(cands):
    return sum(1 << CLASS[b] for b in cands)


def _both(oracle_mod, dist, logret, nret, horizon, nominal, n_pivot, cands):
    counts, perm = stq.assign_rows(dist, logret, nret, horizon, nominal, n_pivot, _mask(cands))
    Lw = oracle_mod.alloc_lifetime(logret, nret, horizon)
    bits, ocounts, operm = oracle_mod.alloc_assign(dist, Lw, nominal=nominal, n_pivot=n_pivot,
                                                   candidates=cands)
    np.testing.assert_array_equal(counts, ocounts)
    np.testing.assert_array_equal(perm, operm)
    # the budget holds: integer widths sum to at most nominal per integer row
    integer = bits != 16
    assert bits[integer].sum() <= nominal * integer.sum()
    assert int(np.sum(bits == 16)) == n_pivot
    return bits


def _convex_dist(g, hv, d, scale_sigma=1.0):
    """Candidate distortions falling by roughly 4x per 2 bits (a uniform
    quantizer), with per-row scales and multiplicative noise: hulls of 1-4
    vertices, some points above the chord."""
    scale = g.lognormal(0.0, scale_sigma, size=(hv, d, 1))
    widths = np.array([16.0, 8.0, 6.0, 4.0, 2.0])
    base = 4.0 ** (-widths / 2.0)
    noise = g.lognormal(0.0, 0.35, size=(hv, d, 5))
    return scale * base[None, None, :] * noise


def _logret(g, hv, d, n, lo=0.5):
    """Summed log retention over n samples of gates in [lo, 1)."""
    return np.log(g.uniform(lo, 1.0, size=(hv, d, n))).sum(axis=-1)


# 20 random instances: shapes, budgets, candidate sets, pivots, horizons
_RANDOM = [
    # seed, hv, d, nominal, cands, n_pivot, horizon
    (1, 4, 64, 6, (8, 6, 4), 5, 256),
    (2, 4, 64, 4, (8, 6, 4, 2), 5, 256),
    (3, 8, 128, 6, (8, 6, 4), 26, 100),
    (4, 8, 128, 4, (8, 6, 4, 2), 51, 100),
    (5, 2, 16, 6, (8, 6, 4), 0, 1),
    (6, 2, 16, 4, (8, 6, 4, 2), 32, 64),       # every row a pivot
    (7, 3, 32, 2, (8, 6, 4, 2), 3, 64),        # budget at the narrowest width
    (8, 3, 32, 8, (8, 6, 4), 3, 64),           # budget at the widest width
    (9, 4, 64, 6, (8, 6, 4, 2), 7, 4096),
    (10, 4, 64, 4, (8, 4, 2), 2, 128),
    (11, 4, 64, 6, (8, 6), 9, 128),
    (12, 4, 64, 4, (4, 2), 1, 128),
    (13, 16, 128, 6, (8, 6, 4), 13, 100),
    (14, 16, 128, 4, (8, 6, 4, 2), 102, 100),
    (15, 1, 128, 6, (8, 6, 4), 0, 2),
    (16, 1, 128, 4, (8, 6, 4, 2), 127, 2),
    (17, 32, 128, 6, (8, 6, 4), 26, 100),      # the 6-bit serving shape
    (18, 32, 128, 4, (8, 6, 4, 2), 26, 100),
    (19, 5, 48, 6, (8, 6, 4, 2), 11, 33),
    (20, 6, 96, 4, (8, 6, 4, 2), 0, 1000),
    (21, 2, 64, 6, (8, 6, 4), 4, 16),
    (22, 8, 32, 4, (8, 6, 4, 2), 8, 512),
]


@pytest.mark.parametrize("seed,hv,d,nominal,cands,n_pivot,horizon", _RANDOM)
def test_random_instances(oracle_mod, seed, hv, d, nominal, cands, n_pivot, horizon):
    g = np.random.default_rng(7000 + seed)
    n = 24
    dist = _convex_dist(g, hv, d, scale_sigma=1.0 + 0.1 * (seed % 5))
    logret = _logret(g, hv, d, n, lo=0.3 + 0.05 * (seed % 10))
    bits = _both(oracle_mod, dist, logret, float(n), horizon, nominal, n_pivot, cands)
    if nominal not in (min(cands), max(cands)) and n_pivot < hv * d - 8:
        # a real mix: at least two integer widths in use
        assert len(set(bits[bits != 16].tolist())) >= 2


def test_exact_ties_of_duplicated_rows(oracle_mod):
    """Rows copied inside a head and across heads: their pivot scores and
    every hull slope tie exactly, so only the row order decides pivots and
    steps; an odd leftover budget forces a choice among tied rows."""
    g = np.random.default_rng(7101)
    hv, d = 4, 32
    dist = _convex_dist(g, hv, d)
    logret = _logret(g, hv, d, 8)
    src = [(0, 3), (1, 5), (2, 7)]
    for h, i in src:
        for hh in range(hv):
            for ii in (i + 1, i + 9, i + 17):
                dist[hh, ii] = dist[h, i]
                logret[hh, ii] = logret[h, i]
    for n_pivot in (0, 1, 2, 3, 5, 12, 13):
        for nominal, cands in ((6, (8, 6, 4)), (4, (8, 6, 4, 2))):
            _both(oracle_mod, dist, logret, 8.0, 64, nominal, n_pivot, cands)


def test_equal_slopes_across_rows(oracle_mod):
    """Different rows whose hull steps save exactly the same distortion per
    bit (equal differences of exactly representable costs at L_u = horizon):
    the tie goes to the lower row, then the lower width."""
    hv, d = 3, 16
    dist = np.zeros((hv, d, 5))
    # costs at widths 16, 8, 6, 4, 2 (class order); offsets keep the slopes
    base = np.array([0.0, 16.0, 24.0, 40.0, 72.0])
    for h in range(hv):
        for i in range(d):
            dist[h, i] = base + 8.0 * ((h * d + i) % 5)
            dist[h, i, 0] = 0.0
    logret = np.zeros((hv, d))  # retention one: L_u = horizon exactly
    for nominal, cands in ((6, (8, 6, 4)), (4, (8, 6, 4, 2)), (4, (8, 4, 2))):
        for n_pivot in (0, 3, 7):
            _both(oracle_mod, dist, logret, 4.0, 64, nominal, n_pivot, cands)


def test_collinear_and_flat_candidates(oracle_mod):
    """Collinear candidate points (the middle vertex is not on the hull, the
    step jumps two widths), points above the chord, rows where a wider code
    does not lower the distortion (the hull ends early), and rows with zero
    distortion everywhere (no step saves anything)."""
    hv, d = 2, 16
    dist = np.zeros((hv, d, 5))
    for i in range(d):
        kind = i % 4
        if kind == 0:    # collinear: 2 -> 8 in one step of 6 bits
            dist[:, i, 1:] = [10.0, 20.0, 30.0, 40.0]
        elif kind == 1:  # 4 bits above the chord of 2 and 6
            dist[:, i, 1:] = [1.0, 8.0, 30.0, 40.0]
        elif kind == 2:  # nothing below 6 bits helps
            dist[:, i, 1:] = [5.0, 5.0, 12.0, 40.0]
        else:            # zero everywhere
            dist[:, i, 1:] = 0.0
        dist[:, i, 0] = 0.0
    dist[1] *= 3.0
    logret = np.zeros((hv, d))
    for nominal, cands in ((4, (8, 6, 4, 2)), (6, (8, 6, 4)), (4, (8, 4, 2))):
        for n_pivot in (0, 2, 5):
            _both(oracle_mod, dist, logret, 1.0, 16, nominal, n_pivot, cands)


def test_repair_takes_later_steps_that_fit(oracle_mod):
    """A budget the Lagrangian prefix cannot fill: the step at the multiplier
    is a 6-bit jump that does not fit, and the repair takes a smaller step
    that comes after it in the slope order.  Rows 0-5 have collinear points
    (one jump 2 -> 8 saving 100 - i per bit), rows 6-15 steps of 2 bits
    (savings 50, 10, 5 per bit); all costs are exact binary fractions at
    L_u = horizon = 8.  At 4 bits (32 spare bits) five jumps fit (30 bits),
    row 5's does not, and row 6's first step takes the last 2 bits."""
    hv, d = 1, 16
    dist = np.zeros((hv, d, 5))
    logret = np.zeros((hv, d))
    for i in range(d):
        if i < 6:
            s_ = 100.0 - i
            costs = [0.0, 2 * s_, 4 * s_, 6 * s_]  # widths 8, 6, 4, 2
        else:
            costs = [0.0, 10.0, 30.0, 130.0]
        dist[0, i, 1:] = np.array(costs) / 8.0
    bits = _both(oracle_mod, dist, logret, 1.0, 8, 4, 0, (8, 6, 4, 2))
    np.testing.assert_array_equal(bits[0], [8] * 5 + [2, 4] + [2] * 9)
    for nominal in (2, 6, 8):
        _both(oracle_mod, dist, logret, 1.0, 8, nominal, 0, (8, 6, 4, 2))
    for n_pivot in (1, 3):
        _both(oracle_mod, dist, logret, 1.0, 8, 4, n_pivot, (8, 6, 4, 2))


def test_lifetime_weight_regimes(oracle_mod):
    """Retention exactly one (L_u = horizon), close to one (the closed form
    through expm1 against the summed series), strong decay (L_u -> 1), a
    retention above one, and horizon one (L_u = 1 for every row)."""
    g = np.random.default_rng(7105)
    hv, d = 2, 64
    dist = _convex_dist(g, hv, d)
    n = 10.0
    for logret in (np.zeros((hv, d)),
                   np.full((hv, d), -1e-9) * g.uniform(0.5, 1.5, size=(hv, d)),
                   -n * g.uniform(0.0, 3.0, size=(hv, d)),
                   n * g.uniform(0.0, 0.01, size=(hv, d))):
        for horizon in (1, 7, 256, 5000):
            _both(oracle_mod, dist, logret, n, horizon, 4, 3, (8, 6, 4, 2))


def test_rejections():
    lib = stq.lib()
    dist = np.ones((2, 16, 5))
    logret = np.zeros((2, 16))
    counts = np.zeros((2, 5), np.int32)
    perm = np.zeros((2, 16), np.int32)

    def call(hv=2, d=16, nret=1.0, horizon=4, cands=0, nominal=6, piv=0, dist_=dist):
        return lib.stq_assign_rows(hv, d, None if dist_ is None else dist_.ctypes.data,
                                   logret.ctypes.data, nret, horizon, cands, nominal, piv,
                                   counts.ctypes.data, perm.ctypes.data)

    E_ARG = 1
    assert call() == 0
    assert call(dist_=None) == E_ARG
    assert call(hv=0) == E_ARG
    assert call(nret=0.0) == E_ARG
    assert call(nret=float("nan")) == E_ARG
    assert call(horizon=0) == E_ARG
    assert call(nominal=5) == E_ARG
    assert call(cands=0x21) == E_ARG
    assert call(cands=_mask((8, 4))) == E_ARG  # nominal 6 not a candidate
    assert call(piv=-1) == E_ARG
    assert call(piv=33) == E_ARG
    with pytest.raises(ValueError):
        stq.assign_rows(dist.astype(np.float32), logret, 1.0, 4, 6, 0)
    with pytest.raises(ValueError):
        stq.assign_rows(dist[:, :, :4], logret, 1.0, 4, 6, 0)


def _brute_force(cost, widths, budget):
    """min over every choice of one width per row of the summed cost, among
    the choices whose widths fit the budget (exhaustive)."""
    best = np.inf
    n = cost.shape[0]
    idx = np.indices((len(widths),) * n).reshape(n, -1).T
    w = np.asarray(widths)[idx].sum(axis=1)
    tot = cost[np.arange(n)[None, :], idx].sum(axis=1)
    ok = w <= budget
    if ok.any():
        best = tot[ok].min()
    return best


@pytest.mark.parametrize("seed", range(8))
def test_library_optimal_on_convex_instances(seed):
    """The library's assignment alone, checked against exhaustive search
    (no oracle involved): with convex decreasing distortion per row over
    equally spaced widths (2 bits apart), taking the largest weighted saving
    per bit first is optimal, so the result must reach the brute-force
    minimum of sum_i L_i D_i(b_i) for the budget.  L_i is the App. A.3
    lifetime weight, sum over t < H of a_i^(2 t) with a_i the row's mean
    retention, here in closed form (1 - a^(2H)) / (1 - a^2)."""
    g = np.random.default_rng(7100 + seed)
    d, n, H = 7, 5, 40
    # decrements D(2)-D(4) > D(4)-D(6) > D(6)-D(8) > 0, and D(8) >= 0
    dec = np.sort(g.uniform(0.05, 5.0, size=(d, 3)), axis=1)[:, ::-1]
    d8 = g.uniform(0.0, 1.0, size=d)
    dist = np.zeros((1, d, 5))
    dist[0, :, CLASS[8]] = d8
    dist[0, :, CLASS[6]] = d8 + dec[:, 2]
    dist[0, :, CLASS[4]] = d8 + dec[:, 2] + dec[:, 1]
    dist[0, :, CLASS[2]] = d8 + dec[:, 2] + dec[:, 1] + dec[:, 0]
    a = g.uniform(0.6, 0.99, size=d)
    logret = (n * np.log(a))[None, :]
    L = (1.0 - a ** (2 * H)) / (1.0 - a ** 2)
    cls_w = (16, 8, 6, 4, 2)
    cases = 0
    for widths in ((4, 6, 8), (2, 4, 6, 8)):
        cost = np.stack([L * dist[0, :, CLASS[b]] for b in widths], axis=1)
        for nominal in widths[1:-1]:  # the nominal width is one of the candidates
            counts, perm = stq.assign_rows(dist, logret, n, H, nominal, 0, _mask(widths))
            # widths per row from the class counts and the rows in class order
            bits = np.zeros(d, int)
            j = 0
            for k, cnt in enumerate(counts[0]):
                bits[perm[0, j:j + cnt]] = cls_w[k]
                j += cnt
            assert j == d and set(bits) <= set(widths)
            assert bits.sum() <= nominal * d
            got = sum(cost[i, widths.index(int(bits[i]))] for i in range(d))
            best = _brute_force(cost, widths, nominal * d)
            assert got <= best * (1 + 1e-9) + 1e-12, (widths, nominal, got, best)
            cases += 1
    assert cases == 3
