"""GPU parity of the ragged row-class formats (FP16 pivot rows and 8-, 6-, 4-,
2-bit rows; STEPQuant paper App. C.2 Table C1, App. C.3 Table C2) and of the
lifetime-aware calibration (App. A.3, App. C.2) against the CPU oracle,
through the C ABI.

Bars: integer codes >= 99.99 % identical, the rest +-1; row factors within
1e-6 relative (pivot rows exactly 0); a pivot value is the oracle's binary16
or an adjacent one (the GPU rounds its fp32 X, the oracle its double X, and
near a rounding boundary either neighbour is correct); readout within 1e-4
relative L2; refit column factors within 1e-5 relative (against the fit of
the GPU's own codes where a code flipped); candidate distortions within
1e-12 relative (both sides take every rounding decision of the definition in
double; only the summation order differs); summed log retention within 1e-13
relative; the assignment computed by
the library must equal the oracle's assignment of the same statistics
exactly (an integer decision taken from the same doubles).
"""
from __future__ import annotations

import numpy as np
import pytest

from linear_attention_recurrent_rule_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from linear_attention_recurrent_rule_amd import stq  # noqa: E402
from tests import gpu_util as gu  # noqa: E402
from tests import test_gpu_refit as tr  # noqa: E402


def _state(B, hv, hk, d, counts, c, perm, *, fmt=stq.FMT_ALLOC, n_slots=None):
    P = int(counts[:, 0].sum())
    st = stq.State(stq.Geometry(n_slots or B, hv, hk, d, 0, fmt, nominal_bits=8, n_pivot=P))
    st.set_alloc_layout(counts, gu.dev(c), gu.dev(perm))
    torch.cuda.synchronize()
    return st


def _setup(seed, B, hv, d, pivots=1):
    g = wl.rng_for(seed, d)
    counts = wl.random_ragged_counts(hv, d, seed=seed + d, pivots=pivots)
    perm = np.stack([g.permutation(d) for _ in range(hv)]).astype(np.int32)
    c = g.lognormal(0, 0.7, size=(hv, d)).astype(np.float32)
    S = wl.random_states(B, hv, d, seed=seed, outlier_sigma=1.0).astype(np.float32)
    return counts, perm, c, S


def _load(st, pool, r, cs=None):
    st.pool.copy_(gu.dev(pool))
    st.r.copy_(gu.dev(r))
    if cs is not None:
        st.cs.copy_(gu.dev(cs))
    torch.cuda.synchronize()


def _compare(gpu_pool, gpu_r, ref_pool, ref_r, counts, d, label, *, o=None, ref_o=None,
             pivot_err=None, t_exact=None):
    """pivot_err (optional, [B][Hv][d][d] in physical row order): an absolute
    allowance added to the one-ulp bar of each pivot value, for values formed
    by cancellation, where the fp32 evaluation error of the terms exceeds
    half an ulp of the binary16 result.  t_exact (optional, the oracle's exact
    code values in physical rows): a differing integer code must then sit
    within gu.TIE_WINDOW of a rounding boundary, in place of the bar on the
    share of identical codes."""
    zg, hg, cls = wl.unpack_ragged(gpu_pool, counts, d)
    zr, hr, _ = wl.unpack_ragged(ref_pool, counts, d)
    ints = np.broadcast_to(cls[None, :, :, None] != 0, zg.shape)
    diff = np.abs(zg - zr)[ints]
    match = float(np.mean(diff == 0)) if diff.size else 1.0
    if t_exact is None:
        assert match >= gu.CODE_MATCH_MIN, f"{label}: codes identical {match:.6f}"
    else:
        t = np.broadcast_to(t_exact, zg.shape)[ints][diff != 0]
        off = np.abs(t - np.floor(t) - 0.5)
        assert off.size == 0 or off.max() <= gu.TIE_WINDOW, \
            f"{label}: a code differs away from a tie ({off.max():.3g}, match {match:.6f})"
    assert diff.size == 0 or diff.max() <= 1, f"{label}: code differs by {diff.max()}"
    piv = cls[None] == 0
    rows_int = np.broadcast_to(~piv, gpu_r.shape)
    rel = np.abs(gpu_r[rows_int].astype(np.float64) - ref_r[rows_int]) / np.abs(ref_r[rows_int])
    assert rel.size == 0 or rel.max() <= gu.R_RTOL, f"{label}: r rel {rel.max():.3g}"
    assert np.all(gpu_r[np.broadcast_to(piv, gpu_r.shape)] == 0.0), f"{label}: pivot r"
    hpiv = np.broadcast_to(cls[None, :, :, None] == 0, hg.shape)
    va = hg[hpiv].view(np.float16).astype(np.float64)
    vb = hr[hpiv].view(np.float16).astype(np.float64)
    step = np.spacing(np.maximum(np.abs(va), np.abs(vb)).astype(np.float16)).astype(np.float64)
    if pivot_err is not None:
        step = step + pivot_err[hpiv]
    hd = np.abs(va - vb)
    assert hd.size == 0 or np.all(hd <= step), f"{label}: pivot value off by more than 1 ulp"
    stats = dict(code_match=match, max_r_rel=float(rel.max()) if rel.size else 0.0,
                 pivot_exact=float(np.mean(hd == 0)) if hd.size else 1.0)
    if o is not None:
        num = np.sqrt(np.sum((o.astype(np.float64) - ref_o) ** 2, axis=-1))
        den = np.sqrt(np.sum(ref_o.astype(np.float64) ** 2, axis=-1))
        rel_o = np.where(den > 0, num / np.where(den > 0, den, 1), num)
        assert rel_o.max() <= 1e-4, f"{label}: readout rel L2 {rel_o.max():.3g}"
        stats["max_o_rel_l2"] = float(rel_o.max())
    return stats


U = 2.0 ** -24  # fp32 unit roundoff
# fp32 roundings that the column sums u~ (and so e) may carry, relative to the
# sum of the magnitudes of their terms: up to 32 in the matrix-core products
# of a wave (16 products of a row group into the accumulator per product,
# two chained products), 2 joining the three coefficient parts, 4 joining the
# waves, 2 adding the pivot rows; the d < 128 kernel's chain (8 per-lane
# FMAs, at most 16 row-group partials) is shorter
SUM_ROUNDINGS = 40


def pivot_allowance(pool, r, counts, perm, c, k, v, beta, X, d, *, alpha=None, gate=None):
    """Per pivot value [B][Hv][d][d] (physical rows; c the column factors per
    head [Hv][d] or per state [B][Hv][d]): a bound on the distance
    between the kernel's fp32 value of X_ij and the exact one, from its
    rounding chain.  With T1 = g_i h_ij (the gated old value, g the gate:
    alpha or the row gate d_i) and T2 = X_ij - T1 (the delta write):
      * the d = 128 kernel forms z = h fl(rcp(c)) (rcp within 1 ulp = 2u,
        the product u), y = fl(P z + e) with P = ar / bk refined to within
        1.5u, ar = fl(a g) (u when a row gate multiplies), bk = fl(b k), and
        X = fl(c fl(bk y)): the old value carries the roundings of rcp,
        z, ar, P, y, bk y and c (.), at most 7.5u |T1|; the delta write those
        of bk, y, bk y and c (.), 4u |T2|;
      * the d < 128 kernel forms x = fl(ar z + fl(bk e)), X = fl(c x): 6u |T1|
        and 4u |T2|, within the same bound;
      * e itself: e = (v - a u_pivots) / c - a u, the quotient within 1.5u of
        |v / c|, the final FMA u |e|, and the column sums within
        SUM_ROUNDINGS u of the sum of the magnitudes of their terms
        (g_i r_i k_i z_ij for integer rows, g_i k_i h_ij / c_j for pivots),
        scaled by a; it enters X through c bk.
    The oracle's binary16 value of the exact X and the kernel's of its fp32
    value then differ by at most one binary16 ulp plus this bound."""
    codes, hbits, cls = wl.unpack_ragged(pool, counts, d)
    B, hv = r.shape[:2]
    G = hv // k.shape[1]
    kh = k.astype(np.float64)[:, np.arange(hv) // G, :]            # [B][Hv][d] logical
    kp = np.take_along_axis(kh, np.broadcast_to(perm[None], kh.shape), axis=2)  # physical
    if gate is not None:
        gp = np.take_along_axis(gate.astype(np.float64), np.broadcast_to(perm[None], kh.shape), axis=2)
        a = np.ones((B, hv))
    else:
        gp = np.ones_like(kp)
        a = alpha.astype(np.float64)
    piv = (cls == 0)[None, :, :, None]                               # [1][Hv][d][1]
    h = hbits.view(np.float16).astype(np.float64)
    # c per head [Hv][d], or per state [B][Hv][d] (the refit format)
    cb = c.astype(np.float64) if c.ndim == 3 else c.astype(np.float64)[None]
    cc = cb[:, :, None, :]                                           # [.][Hv][1][d]
    rr = r.astype(np.float64)[..., None]
    coef = np.where(piv, gp[..., None] * kp[..., None] / cc, gp[..., None] * rr * kp[..., None])
    val = np.where(piv, h, codes.astype(np.float64))
    terms = coef * val                                              # [B][Hv][d][d]
    u_sum = terms.sum(axis=2)                                       # [B][Hv][d] per column
    u_abs = np.abs(terms).sum(axis=2)
    vc = v.astype(np.float64) / cb
    e = vc - a[..., None] * u_sum
    de = U * (1.5 * np.abs(vc) + np.abs(e) + SUM_ROUNDINGS * a[..., None] * u_abs)
    Xp = np.take_along_axis(X, perm[None, :, :, None], axis=2)        # physical rows
    t1 = a[..., None, None] * gp[..., None] * h
    t2 = Xp - t1
    cbk = np.abs(cc * beta.astype(np.float64)[..., None, None] * kp[..., None])
    return U * (7.5 * np.abs(t1) + 4.0 * np.abs(t2)) + cbk * de[:, :, None, :]


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_alloc_pack_dequant_parity(oracle_mod, d):
    B, hv, hk = 3, 4, 2
    print(f"[case] ragged pack d={d}", flush=True)
    counts, perm, c, S = _setup(4001, B, hv, d, pivots=2)
    st = _state(B, hv, hk, d, counts, c, perm)
    st.pack(gu.dev(S))
    torch.cuda.synchronize()
    pool = st.pool.cpu().numpy()
    r = st.r.cpu().numpy()
    ref_pool, ref_r = oracle_mod.alloc_pack(S.astype(np.float64), counts, perm, c, st.slot_bytes)
    print(_compare(pool, r, ref_pool, ref_r, counts, d, f"pack d={d}"))
    # dequant of the GPU's own pool: at most two fp32 roundings of r c z
    got = st.dequant().cpu().numpy()
    ref = oracle_mod.alloc_dequant(pool, r, counts, perm, c=c)
    np.testing.assert_allclose(got, ref, rtol=2.5e-7, atol=1e-30)


@pytest.mark.parametrize("d,dtype,gated", [(16, "f32", False), (32, "bf16", False),
                                           (64, "f32", True), (128, "bf16", False),
                                           (128, "bf16", True), (128, "f32", False)])
def test_alloc_step_parity(oracle_mod, d, dtype, gated):
    B, hv, hk = 5, 8, 4
    print(f"[case] ragged step d={d} {dtype} gated={gated}", flush=True)
    counts, perm, c, S = _setup(4002, B, hv, d, pivots=3)
    st = _state(B, hv, hk, d, counts, c, perm)
    pool, r = oracle_mod.alloc_pack(S.astype(np.float64), counts, perm, c, st.slot_bytes)
    _load(st, pool, r)
    x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=4002, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    if gated:
        gate = wl.draw_gate(B, hv, d, seed=4002, step=0)
        o = st.decode_step_gated(q, k, v, gu.dev(gate), b)
        ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, None, x.beta, c=c,
                                    gate=gate)
    else:
        o = st.decode_step(q, k, v, a, b)
        ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, x.alpha, x.beta, c=c)
    torch.cuda.synchronize()
    print(_compare(st.pool.cpu().numpy(), st.r.cpu().numpy(), ref["pool"], ref["r"], counts, d,
                   f"step d={d}", o=o.cpu().numpy(), ref_o=ref["o"]))


def test_alloc_trajectory_per_step(oracle_mod):
    """Eight steps with the oracle's state fed back each time."""
    B, hv, hk, d = 3, 4, 4, 128
    counts, perm, c, S = _setup(4003, B, hv, d, pivots=2)
    st = _state(B, hv, hk, d, counts, c, perm)
    pool, r = oracle_mod.alloc_pack(S.astype(np.float64), counts, perm, c, st.slot_bytes)
    for t in range(8):
        print(f"[case] ragged trajectory step {t}", flush=True)
        _load(st, pool, r)
        x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=4003, step=t)
        q, k, v, a, b = gu.inputs_to_device(x)
        o = st.decode_step(q, k, v, a, b)
        ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, x.alpha, x.beta, c=c)
        torch.cuda.synchronize()
        _compare(st.pool.cpu().numpy(), st.r.cpu().numpy(), ref["pool"], ref["r"], counts, d,
                 f"t={t}", o=o.cpu().numpy(), ref_o=ref["o"])
        pool, r = ref["pool"], ref["r"]


@pytest.mark.parametrize("d,gated", [(128, False), (128, True), (64, False)])
def test_alloc_step_parity_sparse_keys(oracle_mod, d, gated):
    """Keys with about a quarter of their entries exactly zero: rows whose
    b k_i vanishes (pivot and integer rows alike) take the other form of the
    update inside units whose other rows take the usual one."""
    from tests.test_gpu_parity import _sparse_keys

    B, hv, hk = 5, 8, 4
    print(f"[case] ragged sparse keys d={d} gated={gated}", flush=True)
    counts, perm, c, S = _setup(4030, B, hv, d, pivots=3)
    st = _state(B, hv, hk, d, counts, c, perm)
    pool, r = oracle_mod.alloc_pack(S.astype(np.float64), counts, perm, c, st.slot_bytes)
    _load(st, pool, r)
    x = _sparse_keys(wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=4030, step=0), 4031 + d)
    assert np.any(x.k == 0.0)
    q, k, v, a, b = gu.inputs_to_device(x)
    if gated:
        gate = wl.draw_gate(B, hv, d, seed=4030, step=0)
        o = st.decode_step_gated(q, k, v, gu.dev(gate), b)
        ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, None, x.beta, c=c,
                                    gate=gate, want_X=True)
    else:
        o = st.decode_step(q, k, v, a, b)
        ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, x.alpha, x.beta, c=c,
                                    want_X=True)
    torch.cuda.synchronize()
    # rows with k_i = 0 are only rescaled: their code values cluster at halves
    with np.errstate(divide="ignore", invalid="ignore"):
        t = gu.exact_code_values(ref["X"], ref["r"], c, perm)  # (inf on pivot rows: unused)
    print(_compare(st.pool.cpu().numpy(), st.r.cpu().numpy(), ref["pool"], ref["r"], counts, d,
                   f"sparse keys d={d}", o=o.cpu().numpy(), ref_o=ref["o"], t_exact=t))


@pytest.mark.parametrize("d,gated", [(128, False), (64, True)])
def test_alloc_refit_step_parity(oracle_mod, d, gated):
    B, hv, hk = 4, 4, 2
    print(f"[case] ragged refit d={d} gated={gated}", flush=True)
    counts, perm, c, S = _setup(4004, B, hv, d, pivots=2)
    g = wl.rng_for(4004, 1)
    w2 = (g.uniform(0.05, 1.0, size=(hv, d)) ** 0.5).astype(np.float32)
    st = _state(B, hv, hk, d, counts, c, perm, fmt=stq.FMT_ALLOC_REFIT)
    st.w2.copy_(gu.dev(w2))
    pool, r, cs = oracle_mod.alloc_pack(S.astype(np.float64), counts, perm, c, st.slot_bytes,
                                        w2=w2, refit=True)
    _load(st, pool, r, cs)
    x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=4004, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    kw = {}
    if gated:
        gate = wl.draw_gate(B, hv, d, seed=4004, step=0)
        o = st.decode_step_gated(q, k, v, gu.dev(gate), b)
        kw = dict(gate=gate)
        alpha = None
    else:
        o = st.decode_step(q, k, v, a, b)
        alpha = x.alpha
    ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, alpha, x.beta, cs=cs, w2=w2,
                                want_X=True, **kw)
    torch.cuda.synchronize()
    gp, gr = st.pool.cpu().numpy(), st.r.cpu().numpy()
    stats = _compare(gp, gr, ref["pool"], ref["r"], counts, d, "refit", o=o.cpu().numpy(),
                     ref_o=ref["o"])
    zg, _, cls = wl.unpack_ragged(gp, counts, d)
    zr, _, _ = wl.unpack_ragged(ref["pool"], counts, d)
    stats["max_cs_rel"] = tr._compare_cs(st.cs.cpu().numpy(), ref["cs"], "ragged refit", X=ref["X"],
                                         z=zg, zref=zr, r=gr, perm=perm, w2=w2, cs_old=cs)
    print(stats)


def test_alloc_decode_into_matches_in_place(oracle_mod):
    B, hv, hk, d = 3, 4, 2, 64
    counts, perm, c, S = _setup(4005, B, hv, d, pivots=1)
    src = _state(B, hv, hk, d, counts, c, perm)
    dst = _state(B, hv, hk, d, counts, c, perm)
    ref_st = _state(B, hv, hk, d, counts, c, perm)
    pool, r = oracle_mod.alloc_pack(S.astype(np.float64), counts, perm, c, src.slot_bytes)
    _load(src, pool, r)
    _load(ref_st, pool, r)
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=4005, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    o1 = src.decode_step_into(dst, q, k, v, a, b)
    o2 = ref_st.decode_step(q, k, v, a, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(dst.pool, ref_st.pool) and torch.equal(dst.r, ref_st.r)
    np.testing.assert_array_equal(src.pool.cpu().numpy(), pool)  # source untouched


@pytest.mark.parametrize("d,gated", [(64, False), (128, True)])
def test_alloc_calibration_and_assignment(oracle_mod, d, gated):
    """Column factors, candidate distortions and retention on the GPU against
    the oracle; the library's assignment against the oracle's assignment of
    the same statistics; then a packed step on the chosen layout."""
    hv, hk, B, steps = 4, 2, 6, 3
    print(f"[case] ragged calibration d={d} gated={gated}", flush=True)
    P = 5
    st = stq.State(stq.Geometry(B, hv, hk, d, 0, stq.FMT_ALLOC, nominal_bits=6, n_pivot=P))
    st.calibrate(None, stq.CAL_RESET)
    records = [wl.random_states(B, hv, d, seed=4100 + t, outlier_sigma=1.0).astype(np.float32)
               for t in range(steps)]
    for rec in records:
        st.calibrate(gu.dev(rec), stq.CAL_COLS)
    st.calibrate(None, stq.CAL_FINALIZE)
    torch.cuda.synchronize()
    allrec = np.concatenate(records)
    cmax = np.max(np.abs(allrec), axis=(0, 2))
    c_expect = np.where(cmax > 0, cmax, 1.0).astype(np.float32)
    np.testing.assert_array_equal(st.c.cpu().numpy(), c_expect)
    for rec in records:
        st.calibrate(gu.dev(rec), stq.CAL_DIST)
    dist_ref = np.zeros((hv, d, 5))
    oracle_mod.alloc_distortion(allrec.astype(np.float64), c_expect, dist_ref)
    logret_ref = np.zeros((hv, d))
    for t in range(steps):
        x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=4101, step=t, alpha_lo=0.5)
        if gated:
            gate = wl.draw_gate(B, hv, d, seed=4101, step=t)
            st.calibrate_retention(gate=gu.dev(gate))
            logret_ref += np.sum(np.log(gate.astype(np.float64)), axis=0)
        else:
            st.calibrate_retention(alpha=gu.dev(x.alpha))
            logret_ref += np.sum(np.log(x.alpha.astype(np.float64)), axis=0)[:, None]
    torch.cuda.synchronize()
    dist = st.dist.cpu().numpy()
    np.testing.assert_allclose(dist, dist_ref, rtol=1e-12, atol=0)
    logret = st.logret.cpu().numpy()
    np.testing.assert_allclose(logret, logret_ref, rtol=1e-13, atol=0)
    assert np.all(st.nret.cpu().numpy() == B * steps)
    H = 256
    st.allocate(H)
    torch.cuda.synchronize()
    Lw = oracle_mod.alloc_lifetime(logret, float(B * steps), H)
    bits, counts, perm = oracle_mod.alloc_assign(dist, Lw, nominal=6, n_pivot=P,
                                                 candidates=(8, 6, 4))
    lay = st.layout.cpu().numpy()
    np.testing.assert_array_equal(lay[:, :5], counts)
    np.testing.assert_array_equal(st.perm.cpu().numpy(), perm)
    np.testing.assert_array_equal(lay[:, 5], wl.ragged_segments(counts, d))
    print("widths used:", {b: int(np.sum(bits == b)) for b in (16, 8, 6, 4)})
    # a step on the chosen layout
    S = records[0]
    st.pack(gu.dev(S))
    torch.cuda.synchronize()
    pool, r = st.pool.cpu().numpy(), st.r.cpu().numpy()
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=4102, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    o = st.decode_step(q, k, v, a, b)
    torch.cuda.synchronize()
    ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, x.alpha, x.beta,
                                c=c_expect)
    _compare(st.pool.cpu().numpy(), st.r.cpu().numpy(), ref["pool"], ref["r"], counts, d,
             "allocated", o=o.cpu().numpy(), ref_o=ref["o"])
