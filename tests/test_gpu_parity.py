"""GPU parity of the HIP decode path against the CPU oracle, through the C ABI.

Bar (per step, same input state): >= 99.99 % of codes identical and the rest
within +-1, every row factor within 1e-6 relative, the readout within 1e-4
relative L2 per (sequence, head).  Inputs are seeded and synthetic; no input
or expected value comes from the HIP path (per-step trajectory checks feed the
oracle's own state to the GPU, never the other way round).
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


def _one_step(oracle_mod, B, hv, hk, d, n8, *, dtype, seed, nthreads=8, c_one=False,
              identity_perm=False, fmt=stq.FMT_MIXED48):
    print(f"[case] B={B} hv={hv} hk={hk} d={d} n8={n8} dtype={dtype} seed={seed} fmt={fmt}",
          flush=True)
    ps = wl.random_packed_state(B, hv, d, n8, seed=seed, c_one=c_one, identity_perm=identity_perm)
    x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=seed, step=0)
    st = gu.make_state(B, hv, hk, d, n8, fmt=fmt)
    gu.load_packed(st, ps)
    o = gu.gpu_step(st, x)
    p8, p4, r = gu.read_packed(st)
    ref = gu.oracle_step_on(oracle_mod, ps, x, nthreads)
    return gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d,
                           label=f"d={d} n8={n8} {dtype}"), ps, (p8, p4, r, o)


@pytest.mark.parametrize("d,n8,B,hv,hk", [
    (16, 16, 1, 1, 1),     # tiny: all rows 8-bit
    (16, 8, 7, 3, 1),      # ragged: 21 units over 64-unit workgroups
    (32, 13, 5, 4, 2),     # n8 not a multiple of the lane-group height
    (32, 0, 4, 2, 2),      # all rows 4-bit
    (64, 32, 8, 4, 4),     # small mixed
    (64, 64, 3, 4, 1),     # all 8-bit, GQA 4
    (128, 64, 6, 32, 16),  # serving shape, 6-bit mix
    (128, 16, 5, 32, 16),  # 4.5-bit mix
    (128, 128, 2, 4, 2),   # all 8-bit
    (128, 0, 2, 4, 2),     # all 4-bit
    (128, 37, 3, 2, 1),    # ragged split (read at run time; one slot straddles it)
    (128, 3, 4, 8, 4),     # runtime split straddling the first slot
    (128, 124, 2, 4, 2),   # runtime split on a 4-row boundary (no straddle)
    (128, 125, 3, 32, 16), # runtime split straddling the last slot
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_parity_random_state(oracle_mod, d, n8, B, hv, hk, dtype):
    stats, *_ = _one_step(oracle_mod, B, hv, hk, d, n8, dtype=dtype, seed=1000 + d + n8)
    print(stats)


def test_int8row_format_parity(oracle_mod):
    """INT8ROW (n8 = d, c = 1, identity order) matches the oracle's mixed step
    with the same settings (the uniform rowwise-absmax INT8 baseline)."""
    stats, *_ = _one_step(oracle_mod, 4, 32, 16, 128, 128, dtype="bf16", seed=77, c_one=True,
                          identity_perm=True, fmt=stq.FMT_INT8ROW)
    print(stats)


def test_fixed_point_on_gpu(oracle_mod):
    """alpha = 1, beta = 0 with every row spanning its full code range: the
    state is a fixed point, so the codes come back unchanged and r within 1e-6
    (Eq. (1) with D = I and no write)."""
    B, hv, hk, d, n8 = 3, 8, 4, 128, 64
    print(f"[case] fixed point B={B} hv={hv} d={d} n8={n8}", flush=True)
    ps = wl.random_packed_state(B, hv, d, n8, seed=5, full_rows=True)
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=5, step=0)
    x.alpha[:] = 1.0
    x.beta[:] = 0.0
    st = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(st, ps)
    gu.gpu_step(st, x)
    p8, p4, r = gu.read_packed(st)
    np.testing.assert_array_equal(p8, ps.pool8)
    np.testing.assert_array_equal(p4, ps.pool4)
    np.testing.assert_allclose(r, ps.r, rtol=1e-6, atol=0)


def test_zero_state_first_step(oracle_mod):
    """From the empty state (codes 0, r = 2^-126) the GPU step equals the
    oracle's (which is pinned to the closed form X = beta k v^T)."""
    B, hv, hk, d, n8 = 4, 4, 2, 64, 32
    st = gu.make_state(B, hv, hk, d, n8)
    g = wl.rng_for(9, 9)
    c = g.lognormal(0, 0.5, size=(hv, d)).astype(np.float32)
    perm = np.stack([g.permutation(d) for _ in range(hv)]).astype(np.int32)
    st.set_calibration(gu.dev(c), gu.dev(perm))
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=9, step=0)
    o = gu.gpu_step(st, x)
    p8, p4, r = gu.read_packed(st)
    ps = wl.PackedState(np.zeros((B, hv, n8, d), np.int8),
                        np.zeros((B, hv, d - n8, d // 2), np.uint8),
                        np.full((B, hv, d), 2.0 ** -126, np.float32), c, perm, n8)
    ref = gu.oracle_step_on(oracle_mod, ps, x)
    print(gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d))


def _sparse_keys(x: wl.StepInputs, seed: int, frac: float = 0.25) -> wl.StepInputs:
    """The same inputs with about `frac` of the key entries exactly zero."""
    import dataclasses

    zero = wl.rng_for(seed, 77).random(x.k.shape) < frac
    k = np.where(zero, np.float32(0.0), x.k).astype(np.float32)
    kb = None if x.k_bits is None else np.where(zero, 0, x.k_bits).astype(x.k_bits.dtype)
    return dataclasses.replace(x, k=k, k_bits=kb)


@pytest.mark.parametrize("d,n8,dtype", [(128, 64, "bf16"), (128, 40, "f32"), (64, 32, "bf16"),
                                        (32, 13, "f32")])
def test_step_parity_sparse_keys(oracle_mod, d, n8, dtype):
    """Keys with exact zeros: a row whose b k_i vanishes takes the other form
    of the update (no delta write, the decayed row alone), inside units
    whose other rows take the usual one."""
    B, hv, hk = 6, 8, 4
    print(f"[case] sparse keys d={d} n8={n8} {dtype}", flush=True)
    ps = wl.random_packed_state(B, hv, d, n8, seed=1300 + d + n8)
    x = _sparse_keys(wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=1301, step=0), 1302 + d)
    assert np.any(x.k == 0.0) and np.any(x.k != 0.0)
    st = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(st, ps)
    o = gu.gpu_step(st, x)
    p8, p4, r = gu.read_packed(st)
    ref = oracle_mod.step(ps.pool8, ps.pool4, ps.r, ps.c, ps.perm, x.q, x.k, x.v, x.alpha,
                          x.beta, n8=n8, nthreads=8, want_X=True)
    # a row with k_i = 0 is only rescaled, so where its codes do not span
    # the range its new code values cluster at halves: the tie-aware check
    t = gu.exact_code_values(ref["X"], ref["r"], ps.c, ps.perm)
    print(gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=d,
                          label=f"sparse keys d={d} n8={n8}", t_exact=t))


@pytest.mark.parametrize("d,n8,hv,hk", [(64, 32, 4, 2), (128, 64, 8, 4), (128, 16, 32, 16)])
def test_slot_mapping_and_untouched_slots(oracle_mod, d, n8, hv, hk):
    """A batch addressing a permuted subset of slots updates exactly those
    slots; the others keep their bytes."""
    n_slots, B = 10, 4
    ps_all = wl.random_packed_state(n_slots, hv, d, n8, seed=31)
    st = gu.make_state(B, hv, hk, d, n8, n_slots=n_slots)
    gu.load_packed(st, ps_all)
    slots = np.array([7, 2, 9, 4], np.int32)
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=31, step=0)
    o = gu.gpu_step(st, x, slots_t=gu.dev(slots))
    p8, p4, r = gu.read_packed(st)
    sub = wl.PackedState(ps_all.pool8[slots], ps_all.pool4[slots], ps_all.r[slots], ps_all.c,
                         ps_all.perm, n8)
    ref = gu.oracle_step_on(oracle_mod, sub, x)
    gu.compare_step(dict(pool8=p8[slots], pool4=p4[slots], r=r[slots], o=o), ref, n8=n8, d=d)
    rest = np.setdiff1d(np.arange(n_slots), slots)
    np.testing.assert_array_equal(p8[rest], ps_all.pool8[rest])
    np.testing.assert_array_equal(p4[rest], ps_all.pool4[rest])
    np.testing.assert_array_equal(r[rest], ps_all.r[rest])


@pytest.mark.parametrize("d,n8,hv,hk", [(32, 16, 2, 2), (128, 64, 4, 2)])
def test_out_of_range_slot_is_skipped(oracle_mod, d, n8, hv, hk):
    """A slot outside [0, n_slots) leaves the pool untouched and fills o with NaN."""
    n_slots, B = 4, 2
    ps = wl.random_packed_state(n_slots, hv, d, n8, seed=41)
    st = gu.make_state(B, hv, hk, d, n8, n_slots=n_slots)
    gu.load_packed(st, ps)
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=41, step=0)
    o = gu.gpu_step(st, x, slots_t=gu.dev(np.array([1, 17], np.int32)))
    p8, p4, r = gu.read_packed(st)
    assert np.all(np.isnan(o[1])) and np.all(np.isfinite(o[0]))
    for s in (0, 2, 3):
        np.testing.assert_array_equal(p8[s], ps.pool8[s])
        np.testing.assert_array_equal(p4[s], ps.pool4[s])
        np.testing.assert_array_equal(r[s], ps.r[s])
    # and the live sequence still matches the oracle
    sub = wl.PackedState(ps.pool8[[1]], ps.pool4[[1]], ps.r[[1]], ps.c, ps.perm, n8)
    x1 = wl.StepInputs(x.q[[0]], x.k[[0]], x.v[[0]], x.alpha[[0]], x.beta[[0]], x.dtype)
    ref = gu.oracle_step_on(oracle_mod, sub, x1)
    gu.compare_step(dict(pool8=p8[[1]], pool4=p4[[1]], r=r[[1]], o=o[[0]]), ref, n8=n8, d=d)


def test_repeated_slot_rejected_with_debug_check(monkeypatch):
    """With STQ_CHECK_SLOTS set, a repeated slot is rejected on the host before
    anything is queued (decode and pack); without it the call is accepted (the
    precondition is the caller's).  Slots out of range stay allowed."""
    d, n8, hv, hk, n_slots = 64, 32, 2, 1, 4
    ps = wl.random_packed_state(n_slots, hv, d, n8, seed=43)
    st = gu.make_state(n_slots, hv, hk, d, n8)
    gu.load_packed(st, ps)
    x = wl.draw_inputs(2, hk, hv, d, dtype="f32", seed=43, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    dup = gu.dev(np.array([2, 2], np.int32))
    monkeypatch.setenv("STQ_CHECK_SLOTS", "1")
    with pytest.raises(stq.StqError, match="STQ_E_ARG"):
        st.decode_step(q, k, v, a, b, slots=dup)
    S = gu.dev(np.zeros((2, hv, d, d), np.float32))
    with pytest.raises(stq.StqError, match="STQ_E_ARG"):
        st.pack(S, slots=dup)
    st.decode_step(q, k, v, a, b, slots=gu.dev(np.array([3, 17], np.int32)))  # 17: skipped
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.pool8[2].cpu().numpy(), ps.pool8[2])  # nothing ran on 2
    monkeypatch.delenv("STQ_CHECK_SLOTS")
    st.decode_step(q, k, v, a, b, slots=gu.dev(np.array([0, 1], np.int32)))
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,steps", [("tiny", 64)])
def test_trajectory_per_step_parity(oracle_mod, name, steps):
    """Along the oracle's own trajectory of a workload (S0 packed by the
    oracle), every step run on the GPU from the oracle's state matches the
    oracle's next state."""
    w = wl.WORKLOADS[name]
    S0 = wl.initial_state(w)
    g = wl.rng_for(w.seed, 77)
    if name == "tiny":
        c = np.ones((w.hv, w.d), np.float32)
        perm = np.tile(np.arange(w.d, dtype=np.int32), (w.hv, 1))
    else:
        c = g.lognormal(0, 0.5, size=(w.hv, w.d)).astype(np.float32)
        perm = np.stack([g.permutation(w.d) for _ in range(w.hv)]).astype(np.int32)
    p8, p4, r = oracle_mod.pack(S0, c, perm, n8=w.n8)
    st = gu.make_state(w.B, w.hv, w.hk, w.d, w.n8)
    worst = dict(code_match=1.0, max_r_rel=0.0, max_o_rel_l2=0.0)
    for t in range(steps):
        ps = wl.PackedState(p8, p4, r, c, perm, w.n8)
        x = wl.workload_inputs(w, t)
        gu.load_packed(st, ps)
        o = gu.gpu_step(st, x)
        gp8, gp4, gr = gu.read_packed(st)
        ref = gu.oracle_step_on(oracle_mod, ps, x)
        s = gu.compare_step(dict(pool8=gp8, pool4=gp4, r=gr, o=o), ref, n8=w.n8, d=w.d,
                            label=f"{name} step {t}")
        worst = dict(code_match=min(worst["code_match"], s["code_match"]),
                     max_r_rel=max(worst["max_r_rel"], s["max_r_rel"]),
                     max_o_rel_l2=max(worst["max_o_rel_l2"], s["max_o_rel_l2"]))
        p8, p4, r = ref["pool8"], ref["pool4"], ref["r"]
    print(name, worst)


@pytest.mark.parametrize("d,n8", [(16, 16), (32, 5), (64, 32), (128, 64), (128, 16)])
def test_pack_parity(oracle_mod, d, n8):
    """GPU pack of a given fp32 state vs the oracle's pack."""
    B, hv = 6, 4
    S = wl.random_states(B, hv, d, seed=d + n8, outlier_sigma=1.5)
    g = wl.rng_for(d, n8, 3)
    c = g.lognormal(0, 1, size=(hv, d)).astype(np.float32)
    perm = np.stack([g.permutation(d) for _ in range(hv)]).astype(np.int32)
    st = gu.make_state(B, hv, 1, d, n8)
    st.set_calibration(gu.dev(c), gu.dev(perm))
    st.pack(gu.dev(S))
    p8, p4, r = gu.read_packed(st)
    rp8, rp4, rr = oracle_mod.pack(S, c, perm, n8=n8, nthreads=8)
    zg = wl.unpack_codes(p8.reshape(B, hv, n8, d), p4.reshape(B, hv, d - n8, d // 2)).astype(int)
    zr = wl.unpack_codes(rp8, rp4).astype(int)
    assert np.mean(zg == zr) >= gu.CODE_MATCH_MIN and np.abs(zg - zr).max() <= 1
    np.testing.assert_allclose(r, rr, rtol=1e-6, atol=0)


@pytest.mark.parametrize("d,n8", [(16, 4), (64, 32), (128, 64)])
def test_dequant_parity(oracle_mod, d, n8):
    B, hv = 5, 4
    ps = wl.random_packed_state(B, hv, d, n8, seed=3 * d + n8)
    st = gu.make_state(B, hv, 1, d, n8)
    gu.load_packed(st, ps)
    S = st.dequant().cpu().numpy()
    ref = oracle_mod.dequant(ps.pool8, ps.pool4, ps.r, ps.c, ps.perm, n8=n8)
    # fp32 result of (r c) z: at most two fp32 roundings
    np.testing.assert_allclose(S, ref, rtol=2.5e-7, atol=0)


@pytest.mark.parametrize("d,B,hv,hk", [(16, 3, 2, 1), (64, 4, 4, 2), (128, 4, 32, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp32_state_kernel_parity(oracle_mod, d, B, hv, hk, dtype):
    """The unquantized comparison kernel vs the oracle's unquantized step."""
    S = wl.random_states(B, hv, d, seed=d + B, outlier_sigma=1.0)
    x = wl.draw_inputs(B, hk, hv, d, dtype=dtype, seed=d, step=0)
    st = gu.make_state(B, hv, hk, d, 0, fmt=stq.FMT_FP32)
    st.pack(gu.dev(S))
    o = gu.gpu_step(st, x)
    S_gpu = st.dequant().cpu().numpy().astype(np.float64)
    S_ref = S.astype(np.float64).copy()
    o_ref = oracle_mod.fp_step(S_ref, x.q, x.k, x.v, x.alpha, x.beta, nthreads=8)
    num = np.sqrt(np.sum((S_gpu - S_ref) ** 2, axis=(-1, -2)))
    den = np.sqrt(np.sum(S_ref ** 2, axis=(-1, -2)))
    assert np.all(num <= 1e-6 * den)
    num = np.sqrt(np.sum((o - o_ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(o_ref ** 2, axis=-1))
    assert np.all(num <= 1e-5 * den)


@pytest.mark.parametrize("d,n8,n_rec,hv", [(16, 6, 7, 3), (64, 32, 70, 4), (128, 64, 130, 4)])
def test_calibration_parity(oracle_mod, d, n8, n_rec, hv):
    """GPU calibration vs the oracle's: column factors are maxima of the same
    fp32 values (bit-exact); the 8-bit row set must be a valid top-n8 under the
    oracle's scores (rows whose scores agree to 1e-6 may swap)."""
    rec = wl.random_states(n_rec, hv, d, seed=d + n_rec, outlier_sigma=1.0)
    rec[:, 0, :, 1] = 0.0  # a zero column
    st = gu.make_state(1, hv, 1, d, n8)
    half = n_rec // 2
    st.calibrate(gu.dev(rec[:half]), stq.CAL_RESET | stq.CAL_COLS)
    st.calibrate(gu.dev(rec[half:]), stq.CAL_COLS | stq.CAL_ROWS)
    st.calibrate(None, stq.CAL_FINALIZE)
    torch.cuda.synchronize()
    assert st.calibrated
    c = st.c.cpu().numpy()
    perm = st.perm.cpu().numpy()
    colmax = np.zeros((hv, d))
    rows = np.zeros((hv, d))
    oracle_mod.calib_cols(rec.astype(np.float64), colmax)
    oracle_mod.calib_rows(rec[half:].astype(np.float64), rows)
    c_ref, perm_ref = oracle_mod.calib_finalize(colmax, rows, n8)
    np.testing.assert_array_equal(c, c_ref)
    for h in range(hv):
        assert sorted(perm[h]) == list(range(d))
        assert np.all(np.diff(perm[h][:n8]) > 0) and np.all(np.diff(perm[h][n8:]) > 0)
        if np.array_equal(perm[h], perm_ref[h]):
            continue
        sel = set(perm[h][:n8])
        thresh = np.sort(rows[h])[::-1][n8 - 1] if n8 > 0 else np.inf
        for i in sel.symmetric_difference(set(perm_ref[h][:n8])):
            assert abs(rows[h][i] - thresh) <= 1e-6 * thresh, (h, i)


def test_calibration_deterministic():
    """Two calibrations of the same records give bit-identical results."""
    d, hv, n8 = 128, 8, 64
    rec = gu.dev(wl.random_states(200, hv, d, seed=5, outlier_sigma=1.0))
    outs = []
    for _ in range(2):
        st = gu.make_state(1, hv, 1, d, n8)
        st.calibrate(rec, stq.CAL_RESET | stq.CAL_COLS | stq.CAL_ROWS | stq.CAL_FINALIZE)
        torch.cuda.synchronize()
        outs.append((st.c.cpu().numpy(), st.perm.cpu().numpy(), st.rowscore.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("d,n8,hv,hk", [(32, 16, 2, 2), (64, 32, 4, 2), (128, 64, 8, 4),
                                        (128, 16, 32, 16)])
def test_decode_into_matches_in_place(oracle_mod, d, n8, hv, hk):
    """Reading one pool and writing another gives the in-place step's bytes in
    the addressed slots of the destination, leaves the source untouched and
    the destination's other slots as they were."""
    n_slots, B = 6, 4
    print(f"[case] decode_into d={d} n8={n8} hv={hv} hk={hk}", flush=True)
    ps = wl.random_packed_state(n_slots, hv, d, n8, seed=51)
    junk = wl.random_packed_state(n_slots, hv, d, n8, seed=52)
    src = gu.make_state(B, hv, hk, d, n8, n_slots=n_slots)
    dst = gu.make_state(B, hv, hk, d, n8, n_slots=n_slots)
    ref_st = gu.make_state(B, hv, hk, d, n8, n_slots=n_slots)
    gu.load_packed(src, ps)
    gu.load_packed(ref_st, ps)
    gu.load_packed(dst, wl.PackedState(junk.pool8, junk.pool4, junk.r, ps.c, ps.perm, n8))
    slots = np.array([5, 0, 3, 2], np.int32)
    x = wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=51, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    st_t = gu.dev(slots)
    o_into = src.decode_step_into(dst, q, k, v, a, b, slots=st_t)
    o_in = ref_st.decode_step(q, k, v, a, b, slots=st_t)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o_into.cpu().numpy(), o_in.cpu().numpy())
    s8, s4, sr = gu.read_packed(src)
    np.testing.assert_array_equal(s8, ps.pool8)
    np.testing.assert_array_equal(s4, ps.pool4)
    np.testing.assert_array_equal(sr, ps.r)
    d8, d4, dr = gu.read_packed(dst)
    i8, i4, ir = gu.read_packed(ref_st)
    np.testing.assert_array_equal(d8[slots], i8[slots])
    np.testing.assert_array_equal(d4[slots], i4[slots])
    np.testing.assert_array_equal(dr[slots], ir[slots])
    rest = np.setdiff1d(np.arange(n_slots), slots)
    np.testing.assert_array_equal(d8[rest], junk.pool8[rest])
    np.testing.assert_array_equal(d4[rest], junk.pool4[rest])
    np.testing.assert_array_equal(dr[rest], junk.r[rest])
    sub = wl.PackedState(ps.pool8[slots], ps.pool4[slots], ps.r[slots], ps.c, ps.perm, n8)
    ref = gu.oracle_step_on(oracle_mod, sub, x)
    gu.compare_step(dict(pool8=d8[slots], pool4=d4[slots], r=dr[slots], o=o_into.cpu().numpy()),
                    ref, n8=n8, d=d)


def test_decode_into_fp32_state():
    """The FP32-state baseline reads one pool and writes the other as well."""
    B, hv, hk, d = 3, 4, 2, 64
    print(f"[case] decode_into fp32 B={B} d={d}", flush=True)
    src = gu.make_state(B, hv, hk, d, 0, fmt=stq.FMT_FP32)
    dst = gu.make_state(B, hv, hk, d, 0, fmt=stq.FMT_FP32)
    ref_st = gu.make_state(B, hv, hk, d, 0, fmt=stq.FMT_FP32)
    S0 = torch.randn(B, hv, d, d, generator=torch.Generator().manual_seed(3)).cuda() * 0.1
    src.s32.copy_(S0)
    ref_st.s32.copy_(S0)
    x = wl.draw_inputs(B, hk, hv, d, dtype="f32", seed=61, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    o1 = src.decode_step_into(dst, q, k, v, a, b)
    o2 = ref_st.decode_step(q, k, v, a, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(src.s32, S0)
    assert torch.equal(dst.s32, ref_st.s32)


def test_small_mixed_pipeline_every_step(oracle_mod):
    """The small mixed workload (B = 8, 4 value heads over 4 key heads, d =
    64, n8 = 32, fp32 inputs) through the library's whole pipeline, each part
    against the oracle:
      1. the calibration trajectory: 32 unquantized steps from S0 on the
         FP32-state kernel against the oracle's fp64 steps (relative L2 of
         each state within 1e-6 per step taken);
      2. the calibration: stq_calibrate with COLS on all 32 records and ROWS
         on the last, then FINALIZE, fed the oracle's records (rounded to
         fp32), must give the oracle's c bit for bit and its row order;
      3. the pack of S0 with that calibration against the oracle's pack;
      4. all T = 256 steps, each run from the oracle's state (never the
         other way round), to the per-step bar.  Worst statistics printed."""
    w = wl.WORKLOADS["small_mixed"]
    B, hv, hk, d, n8 = w.B, w.hv, w.hk, w.d, w.n8
    S0 = wl.initial_state(w)
    print(f"[case] small_mixed pipeline B={B} hv={hv} d={d} n8={n8} T={w.T}", flush=True)
    # 1. calibration trajectory
    fp = gu.make_state(B, hv, hk, d, 0, fmt=stq.FMT_FP32)
    fp.pack(gu.dev(S0))
    S = S0.astype(np.float64)
    records = []
    worst_traj = 0.0
    for t in range(w.calib_steps):
        x = wl.workload_inputs(w, t, calibration=True)
        q, k, v, a, b = gu.inputs_to_device(x)
        fp.decode_step(q, k, v, a, b)
        oracle_mod.fp_step(S, x.q, x.k, x.v, x.alpha, x.beta)
        records.append(S.astype(np.float32))
        got = fp.dequant().cpu().numpy().astype(np.float64)
        rel = np.sqrt(np.sum((got - S) ** 2, axis=(-1, -2)) / np.sum(S ** 2, axis=(-1, -2)))
        assert rel.max() <= 1e-6 * (t + 1), f"calibration step {t}: rel L2 {rel.max():.3g}"
        worst_traj = max(worst_traj, float(rel.max()))
    # 2. calibration on the oracle's records
    colmax = np.zeros((hv, d))
    rowscore = np.zeros((hv, d))
    st = gu.make_state(B, hv, hk, d, n8)
    st.calibrate(None, stq.CAL_RESET)
    for t, rec in enumerate(records):
        last = t == len(records) - 1
        st.calibrate(gu.dev(rec), stq.CAL_COLS | (stq.CAL_ROWS if last else 0))
        oracle_mod.calib_cols(rec, colmax)
        if last:
            oracle_mod.calib_rows(rec, rowscore)
    st.calibrate(None, stq.CAL_FINALIZE)
    torch.cuda.synchronize()
    c, perm = oracle_mod.calib_finalize(colmax, rowscore, n8)
    np.testing.assert_array_equal(st.c.cpu().numpy(), c)
    np.testing.assert_array_equal(st.perm.cpu().numpy(), perm)
    # 3. pack of S0
    st.pack(gu.dev(S0))
    p8, p4, r = oracle_mod.pack(S0, c, perm, n8=n8)
    gp8, gp4, gr = gu.read_packed(st)
    zg = wl.unpack_codes(gp8, gp4).astype(np.int32)
    zr = wl.unpack_codes(p8, p4).astype(np.int32)
    assert np.mean(zg == zr) >= gu.CODE_MATCH_MIN and np.abs(zg - zr).max() <= 1
    np.testing.assert_allclose(gr, r, rtol=gu.R_RTOL, atol=0)
    # 4. every step from the oracle's state
    worst = dict(code_match=1.0, max_r_rel=0.0, max_o_rel_l2=0.0)
    for t in range(w.T):
        ps = wl.PackedState(p8, p4, r, c, perm, n8)
        x = wl.workload_inputs(w, t)
        gu.load_packed(st, ps)
        o = gu.gpu_step(st, x)
        gp8, gp4, gr = gu.read_packed(st)
        ref = gu.oracle_step_on(oracle_mod, ps, x)
        s_ = gu.compare_step(dict(pool8=gp8, pool4=gp4, r=gr, o=o), ref, n8=n8, d=d,
                             label=f"small_mixed step {t + 1}")
        worst = dict(code_match=min(worst["code_match"], s_["code_match"]),
                     max_r_rel=max(worst["max_r_rel"], s_["max_r_rel"]),
                     max_o_rel_l2=max(worst["max_o_rel_l2"], s_["max_o_rel_l2"]))
        p8, p4, r = ref["pool8"], ref["pool4"], ref["r"]
    print(f"small_mixed: calibration trajectory worst rel L2 {worst_traj:.3g}; steps {worst}",
          flush=True)
