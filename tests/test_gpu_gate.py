"""GPU parity of the per-key-row gate (the KDA form of the STEPQuant paper's
Sec. 2.1 Eq. (1), D_t = diag(d); Sec. 6.1, App. C.1) against the CPU oracle,
through the C ABI (stq_decode_step_gated, stq_calibrate_impact_gated).

Bar: as for the scalar gate (>= 99.99 % of codes identical, the rest +-1; r
within 1e-6 relative; readout within 1e-4 relative L2; FP32 state within 1e-6
relative L2; refit column factors within 1e-5 relative; row impact within
1e-10 relative).  The gate is drawn per sequence, value head and logical key
row, so a kernel that indexed it by physical row would fail the comparison.
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


def _gated_gpu(st, x, gate, dst=None):
    q, k, v, _, b = gu.inputs_to_device(x)
    o = st.decode_step_gated(q, k, v, gu.dev(gate), b, dst=dst)
    torch.cuda.synchronize()
    return o.cpu().numpy()


@pytest.mark.parametrize("d,n8,B,hv,hk", [
    (128, 64, 6, 32, 16),  # serving shape, 6-bit mix (d = 128 fast path)
    (128, 16, 5, 8, 8),    # 4.5-bit mix, no GQA (KDA heads)
    (128, 128, 2, 4, 2),   # all 8-bit
    (128, 0, 2, 4, 2),     # all 4-bit
    (128, 37, 3, 2, 1),    # ragged split (generic kernel)
    (64, 32, 8, 4, 4),     # small mixed (generic kernel)
    (32, 13, 5, 4, 2),
    (16, 8, 7, 3, 1),      # ragged: 21 units over 64-unit workgroups
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_step_parity(oracle_mod, d, n8, B, hv, hk, dtype):
    seed = 2000 + d + n8
    print(f"[case] gated step B={B} hv={hv} hk={hk} d={d} n8={n8} {dtype}", flush=True)
    ps = wl.random_packed_state(B, hv, d, n8, seed=seed)
    x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=seed, step=0)
    gate = wl.draw_gate(B, hv, d, seed=seed, step=0)
    st = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(st, ps)
    o = _gated_gpu(st, x, gate)
    p8, p4, r = gu.read_packed(st)
    ref = oracle_mod.step(ps.pool8, ps.pool4, ps.r, ps.c, ps.perm, x.q, x.k, x.v, None, x.beta,
                          n8=n8, nthreads=8, gate=gate)
    print(gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d,
                          label=f"gated d={d} n8={n8} {dtype}"))


def test_gated_step_degenerate_rows(oracle_mod):
    """Rows whose gate is 0 or 1 exactly, and heads with beta = 0.  In a head
    with beta = 0 every row with d_i = 0 becomes exactly zero (codes 0, row
    factor 2^-126, checked exactly); elsewhere one row per unit has d_i = 0
    and is the rank-1 row beta k_i e.  (Many such rows in one head would all
    be copies of one normalised vector, so a single rounding tie of e would
    flip the same code in all of them: one such row keeps the code bar
    meaningful.)  With beta = 0 a row is only rescaled by d_i, so its new codes
    are z q_b / max|z|: every row spans its full code range here, which makes
    them the old codes exactly (a row with max|z| < q_b would meet exact
    real-number ties such as 63 * 127 / 126 = 63.5, decided by rounding order
    alone)."""
    B, hv, hk, d, n8 = 4, 8, 4, 128, 64
    ps = wl.random_packed_state(B, hv, d, n8, seed=2101, full_rows=True)
    x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=2101, step=0)
    gate = wl.draw_gate(B, hv, d, seed=2101, step=0)
    zero_heads = np.zeros((B, hv), bool)
    zero_heads[:, ::3] = True
    x.beta[zero_heads] = 0.0
    gate[:, :, 5] = 0.0
    gate[:, :, 1::7] = 1.0
    zrows = np.zeros((B, hv, d), bool)
    zrows[zero_heads] = (np.arange(d) % 5 == 0)[None, :]
    zrows[:, :, 5] |= zero_heads
    gate[zrows] = 0.0
    st = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(st, ps)
    o = _gated_gpu(st, x, gate)
    p8, p4, r = gu.read_packed(st)
    ref = oracle_mod.step(ps.pool8, ps.pool4, ps.r, ps.c, ps.perm, x.q, x.k, x.v, None, x.beta,
                          n8=n8, nthreads=8, gate=gate)
    print(gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d,
                          label="degenerate gate"))
    z = wl.unpack_codes(p8.reshape(B, hv, n8, d), p4.reshape(B, hv, d - n8, d // 2))
    z0 = wl.unpack_codes(ps.pool8, ps.pool4)
    for b in range(B):
        for h in range(hv):
            phys = zrows[b, h][ps.perm[h]]  # physical rows whose logical row is zero
            assert np.all(z[b, h, phys] == 0)
            assert np.all(r[b, h, phys] == np.float32(2.0 ** -126))
            if zero_heads[b, h]:  # rescaled rows keep their codes
                np.testing.assert_array_equal(z[b, h, ~phys], z0[b, h, ~phys])


def test_gated_int8row_parity(oracle_mod):
    B, hv, hk, d = 4, 32, 32, 128
    ps = wl.random_packed_state(B, hv, d, d, seed=2102, c_one=True, identity_perm=True)
    x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=2102, step=0)
    gate = wl.draw_gate(B, hv, d, seed=2102, step=0)
    st = gu.make_state(B, hv, hk, d, d, fmt=stq.FMT_INT8ROW)
    gu.load_packed(st, ps)
    o = _gated_gpu(st, x, gate)
    p8, p4, r = gu.read_packed(st)
    ref = oracle_mod.step(ps.pool8, ps.pool4, ps.r, ps.c, ps.perm, x.q, x.k, x.v, None, x.beta,
                          n8=d, nthreads=8, gate=gate)
    print(gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=d, d=d,
                          label="gated int8row"))


def test_gated_trajectory_per_step(oracle_mod):
    """Eight gated steps; the GPU is fed the oracle's state at every step."""
    B, hv, hk, d, n8 = 3, 8, 8, 128, 64
    ps = wl.random_packed_state(B, hv, d, n8, seed=2103)
    P8, P4, R = ps.pool8, ps.pool4, ps.r
    st = gu.make_state(B, hv, hk, d, n8)
    for t in range(8):
        print(f"[case] gated trajectory step {t}", flush=True)
        gu.load_packed(st, wl.PackedState(P8, P4, R, ps.c, ps.perm, n8))
        x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=2103, step=t)
        gate = wl.draw_gate(B, hv, d, seed=2103, step=t)
        o = _gated_gpu(st, x, gate)
        p8, p4, r = gu.read_packed(st)
        ref = oracle_mod.step(P8, P4, R, ps.c, ps.perm, x.q, x.k, x.v, None, x.beta, n8=n8,
                              nthreads=8, gate=gate)
        gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d, label=f"t={t}")
        P8, P4, R = ref["pool8"], ref["pool4"], ref["r"]


def test_gated_out_of_place_matches_in_place(oracle_mod):
    B, hv, hk, d, n8 = 4, 8, 4, 128, 64
    ps = wl.random_packed_state(B, hv, d, n8, seed=2104)
    x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=2104, step=0)
    gate = wl.draw_gate(B, hv, d, seed=2104, step=0)
    src = gu.make_state(B, hv, hk, d, n8)
    dst = gu.make_state(B, hv, hk, d, n8)
    ref_st = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(src, ps)
    gu.load_packed(ref_st, ps)
    o1 = _gated_gpu(src, x, gate, dst=dst)
    o2 = _gated_gpu(ref_st, x, gate)
    np.testing.assert_array_equal(o1, o2)
    a8, a4, ar = gu.read_packed(dst)
    b8, b4, br = gu.read_packed(ref_st)
    np.testing.assert_array_equal(a8, b8)
    np.testing.assert_array_equal(a4, b4)
    np.testing.assert_array_equal(ar, br)
    s8, s4, sr = gu.read_packed(src)  # source untouched
    np.testing.assert_array_equal(sr, ps.r)
    np.testing.assert_array_equal(s8, ps.pool8)


@pytest.mark.parametrize("d,B,hv,hk", [(16, 3, 2, 1), (64, 4, 4, 2), (128, 4, 32, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_fp32_state_parity(oracle_mod, d, B, hv, hk, dtype):
    S = wl.random_states(B, hv, d, seed=2200 + d, outlier_sigma=1.0)
    x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=2200 + d, step=0)
    gate = wl.draw_gate(B, hv, d, seed=2200 + d, step=0)
    st = gu.make_state(B, hv, hk, d, 0, fmt=stq.FMT_FP32)
    st.pack(gu.dev(S))
    o = _gated_gpu(st, x, gate)
    S_gpu = st.dequant().cpu().numpy().astype(np.float64)
    S_ref = S.astype(np.float64).copy()
    o_ref = oracle_mod.fp_step(S_ref, x.q, x.k, x.v, None, x.beta, nthreads=8, gate=gate)
    num = np.sqrt(np.sum((S_gpu - S_ref) ** 2, axis=(-1, -2)))
    den = np.sqrt(np.sum(S_ref ** 2, axis=(-1, -2)))
    assert np.all(num <= 1e-6 * den)
    num = np.sqrt(np.sum((o - o_ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(o_ref ** 2, axis=-1))
    assert np.all(num <= 1e-5 * den)


@pytest.mark.parametrize("d,n8,dtype", [(128, 64, "bf16"), (128, 40, "f32"), (64, 32, "f32")])
def test_gated_refit_step_parity(oracle_mod, d, n8, dtype):
    B, hv, hk = 5, 8, 8
    print(f"[case] gated refit d={d} n8={n8} {dtype}", flush=True)
    g = wl.rng_for(2300, n8)
    c, perm, w2 = tr._calibration(g, hv, d)
    S = wl.random_states(B, hv, d, seed=2300 + n8, outlier_sigma=1.0)
    P8, P4, R, CS = oracle_mod.pack_refit(S, c, perm, w2, n8=n8)
    st = tr._refit_state(B, hv, hk, d, n8, c, perm, w2)
    tr._load(st, P8, P4, R, CS)
    x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=2300, step=0)
    gate = wl.draw_gate(B, hv, d, seed=2300, step=0)
    o = _gated_gpu(st, x, gate)
    p8, p4, r = gu.read_packed(st)
    cs = st.cs.cpu().numpy()
    ref = oracle_mod.step_refit(P8, P4, R, CS, perm, w2, x.q, x.k, x.v, None, x.beta, n8=n8,
                                want_X=True, gate=gate)
    stats = gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d,
                            label=f"gated refit n8={n8}")
    stats["max_cs_rel"] = tr._compare_cs(
        cs, ref["cs"], f"gated refit n8={n8}", X=ref["X"], z=wl.unpack_codes(p8, p4),
        zref=wl.unpack_codes(ref["pool8"], ref["pool4"]), r=r, perm=perm, w2=w2, cs_old=CS)
    print(stats)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_impact_parity(oracle_mod, dtype):
    B, hv, hk, d, n8 = 6, 8, 4, 64, 32
    st = gu.make_state(B, hv, hk, d, n8, fmt=stq.FMT_REFIT)
    om = np.zeros((hv, d))
    st.calibrate_impact(None, None, None, None, stq.CAL_RESET)
    for t in range(3):
        x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=2400, step=t)
        gate = wl.draw_gate(B, hv, d, seed=2400, step=t)
        q, k, v, a, b = gu.inputs_to_device(x)
        st.calibrate_impact(q, k, None, b, 0, gate=gu.dev(gate))
        oracle_mod.impact_accumulate(x.q, x.k, None, x.beta, om, hv=hv, gate=gate)
    st.calibrate_impact(None, None, None, None, stq.CAL_FINALIZE)
    torch.cuda.synchronize()
    np.testing.assert_allclose(st.impact.cpu().numpy(), om, rtol=1e-10, atol=0)
    np.testing.assert_allclose(st.w2.cpu().numpy(), oracle_mod.impact_weights(om), rtol=1e-6,
                               atol=0)
