"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every function include/stq.h declares, the layout arithmetic is right, and
every rejection path returns its documented status before anything is queued
(the pointers used here are never dereferenced because validation fails
first)."""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "stq.h"

stq = pytest.importorskip("linear_attention_recurrent_rule_amd.stq")

E_ARG, E_SHAPE, E_UNSUPPORTED, E_SPACE, E_STATE = 1, 2, 3, 4, 5
FAKE = 0x10000000  # an aligned address that validation must reject before use


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(stq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = stq.lib()
    names = _declared_functions()
    assert "stq_decode_step" in names and len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"libstq.so does not export {n}"
    assert lib.stq_abi_version() == 7


def _desc(n_slots=4, hv=4, hk=2, d=64, n8=32, fmt=stq.FMT_MIXED48, dv=None, nominal=0, piv=0):
    return stq.Desc(n_slots, hv, hk, d, d if dv is None else dv, n8, fmt, nominal, piv)


def _bytes(**kw):
    return stq.lib().stq_state_bytes(ctypes.byref(_desc(**kw)))


def _alloc_slot_bytes(hv, d, nominal, piv):
    b = nominal * (hv * d - piv) * d // 8 + 2 * d * piv + 16 * hv
    return (b + 15) // 16 * 16


def _r(n):
    return (n + 255) // 256 * 256


def test_state_bytes_layout_arithmetic():
    # mixed 6-bit, d = 128, 1024 slots x 32 heads (the serving pool sizes)
    S, H, D, n8 = 1024, 32, 128, 64
    expect = (_r(S * H * n8 * D) + _r(S * H * (D - n8) * D // 2) + _r(S * H * D * 4)
              + _r(H * D * 4) * 2 + _r(H * D * 4) + _r(H * D * 8)
              + _r(H * 64 * D * 4) + _r(H * 64 * D * 8))
    assert _bytes(n_slots=S, hv=H, hk=16, d=D, n8=n8) == expect
    # the state itself: 12,800 B per (slot, head) at the 6-bit mix = 6.25 bits/value
    per_unit = n8 * D + (D - n8) * D // 2 + D * 4
    assert per_unit == 12800 and per_unit * 8 / (D * D) == 6.25
    # INT8ROW: codes + r, no calibration buffers
    assert _bytes(n_slots=S, hv=H, hk=16, d=D, n8=D, fmt=stq.FMT_INT8ROW) == (
        _r(S * H * D * D) + _r(S * H * D * 4) + _r(H * D * 4) * 2)
    # FP32 state
    assert _bytes(n_slots=8, hv=4, hk=4, d=64, n8=0, fmt=stq.FMT_FP32) == (
        _r(8 * 4 * 64 * 64 * 4) + _r(4 * 64 * 4) * 2)


@pytest.mark.parametrize("kw", [
    dict(d=48),                       # not compiled
    dict(d=256),                      # not compiled
    dict(d=64, dv=32),                # d_k != d_v
    dict(hv=3, hk=2),                 # Hv % Hk
    dict(n8=65),                      # n8 > d_k
    dict(n8=-1),
    dict(n_slots=0),
    dict(fmt=7),
    dict(fmt=stq.FMT_INT8ROW, n8=32),  # INT8ROW needs n8 = d_k
])
def test_state_bytes_rejects_bad_geometry(kw):
    assert _bytes(**kw) == 0


def test_alloc_state_rejections():
    lib = stq.lib()
    out = stq.CState()
    d = _desc()
    need = lib.stq_state_bytes(ctypes.byref(d))
    assert lib.stq_alloc_state(None, FAKE, need, None, ctypes.byref(out)) == E_ARG
    assert lib.stq_alloc_state(ctypes.byref(d), None, need, None, ctypes.byref(out)) == E_ARG
    assert lib.stq_alloc_state(ctypes.byref(d), FAKE + 16, need, None, ctypes.byref(out)) == E_ARG
    assert lib.stq_alloc_state(ctypes.byref(d), FAKE, need - 1, None, ctypes.byref(out)) == E_SPACE
    assert lib.stq_alloc_state(ctypes.byref(_desc(d=48)), FAKE, need, None,
                               ctypes.byref(out)) == E_UNSUPPORTED
    assert lib.stq_alloc_state(ctypes.byref(_desc(hv=3)), FAKE, need, None,
                               ctypes.byref(out)) == E_SHAPE


def _fake_state(fmt=stq.FMT_MIXED48, calibrated=0, n8=32, d=64, n_slots=4):
    st = stq.CState()
    st.desc = _desc(fmt=fmt, n8=n8, d=d, n_slots=n_slots)
    for i, f in enumerate(("pool8", "pool4", "r", "c", "perm", "colmax", "rowscore",
                           "cal_colpart", "cal_rowpart", "s32")):
        setattr(st, f, FAKE + 0x1000000 * (i + 1))
    st.calibrated = calibrated
    return st


def _decode(st, B=2, dtype=0, slots=None, ptrs=None):
    p = ptrs or [FAKE] * 6
    return stq.lib().stq_decode_step(ctypes.byref(st), slots, B, p[0], p[1], p[2], dtype,
                                     p[3], p[4], p[5], None)


def test_decode_rejections():
    st = _fake_state(calibrated=0)
    assert _decode(st) == E_STATE  # mixed state before calibration
    st = _fake_state(calibrated=1)
    assert _decode(st, B=0) == E_SHAPE
    assert _decode(st, B=5) == E_SHAPE  # more sequences than slots
    assert _decode(st, dtype=2) == E_ARG
    assert _decode(st, ptrs=[FAKE, FAKE, None, FAKE, FAKE, FAKE]) == E_ARG
    assert _decode(st, ptrs=[FAKE + 1, FAKE, FAKE, FAKE, FAKE, FAKE], dtype=1) == E_ARG
    assert _decode(st, slots=FAKE + 2) == E_ARG
    # bf16 readout: the flag combines with an input dtype only; o needs 2-byte
    # alignment with it and 4-byte alignment without it
    assert _decode(st, dtype=stq.OUT_BF16 | 2) == E_ARG
    assert _decode(st, dtype=stq.OUT_BF16 | 0x200) == E_ARG
    assert _decode(st, ptrs=[FAKE] * 5 + [FAKE + 1], dtype=stq.OUT_BF16) == E_ARG
    assert _decode(st, ptrs=[FAKE] * 5 + [FAKE + 2]) == E_ARG
    bad = _fake_state(calibrated=1)
    bad.pool8 = None
    assert _decode(bad) == E_ARG
    bad = _fake_state(calibrated=1)
    bad.desc.n_heads_k = 3
    assert _decode(bad) == E_SHAPE
    assert stq.lib().stq_decode_step(None, None, 1, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE,
                                     None) == E_ARG


def test_pack_dequant_calibrate_rejections():
    lib = stq.lib()
    st = _fake_state(calibrated=0)
    assert lib.stq_pack_state(ctypes.byref(st), FAKE, None, 2, None) == E_STATE
    st = _fake_state(calibrated=1)
    assert lib.stq_pack_state(ctypes.byref(st), None, None, 2, None) == E_ARG
    assert lib.stq_pack_state(ctypes.byref(st), FAKE + 4, None, 2, None) == E_ARG
    assert lib.stq_pack_state(ctypes.byref(st), FAKE, None, 9, None) == E_SHAPE
    assert lib.stq_dequant_state(ctypes.byref(st), None, 0, FAKE, None) == E_SHAPE
    assert lib.stq_dequant_state(ctypes.byref(st), None, 2, None, None) == E_ARG
    assert lib.stq_calibrate(ctypes.byref(st), FAKE, 1, 64, None) == E_ARG  # unknown flag
    assert lib.stq_calibrate(ctypes.byref(st), FAKE, -1, stq.CAL_COLS, None) == E_SHAPE
    assert lib.stq_calibrate(ctypes.byref(st), None, 3, stq.CAL_COLS, None) == E_ARG
    i8 = _fake_state(fmt=stq.FMT_INT8ROW, calibrated=1, n8=64)
    assert lib.stq_calibrate(ctypes.byref(i8), FAKE, 1, stq.CAL_COLS, None) == E_ARG
    assert lib.stq_set_calibration(ctypes.byref(i8), FAKE, FAKE, None) == E_ARG
    assert lib.stq_set_calibration(ctypes.byref(st), None, FAKE, None) == E_ARG


def test_stream_copy_rejections():
    lib = stq.lib()
    assert lib.stq_stream_copy(None, FAKE, 16, None) == E_ARG
    assert lib.stq_stream_copy(FAKE, FAKE + 8, 16, None) == E_ARG
    assert lib.stq_stream_copy(FAKE, FAKE, 15, None) == E_ARG


def test_status_strings():
    lib = stq.lib()
    for s in range(7):
        assert lib.stq_status_str(s).decode().startswith("STQ_")
    assert lib.stq_status_str(99) == b"unknown stq_status"


def test_decode_into_rejections():
    lib = stq.lib()
    src = _fake_state(calibrated=1)
    p = [FAKE] * 6

    def into(a, b, B=2):
        return lib.stq_decode_step_into(a, b, None, B, p[0], p[1], p[2], 0, p[3], p[4], p[5],
                                        None)

    assert into(None, ctypes.byref(src)) == E_ARG
    assert into(ctypes.byref(src), None) == E_ARG
    other = _fake_state(calibrated=1, n8=16)  # different descriptor
    assert into(ctypes.byref(src), ctypes.byref(other)) == E_SHAPE
    other = _fake_state(calibrated=1, n_slots=8)
    assert into(ctypes.byref(src), ctypes.byref(other)) == E_SHAPE
    # a destination pool that overlaps the source pool without being it
    shifted = _fake_state(calibrated=1)
    shifted.pool8 = src.pool8 + 64
    assert into(ctypes.byref(src), ctypes.byref(shifted)) == E_ARG
    shifted = _fake_state(calibrated=1)
    shifted.r = src.r + 4
    assert into(ctypes.byref(src), ctypes.byref(shifted)) == E_ARG
    bad = _fake_state(calibrated=1)
    bad.pool4 = None
    assert into(ctypes.byref(src), ctypes.byref(bad)) == E_ARG
    uncal = _fake_state(calibrated=0)
    assert into(ctypes.byref(uncal), ctypes.byref(src)) == E_STATE
    assert into(ctypes.byref(src), ctypes.byref(src), B=0) == E_SHAPE


def test_refit_layout_and_rejections():
    lib = stq.lib()
    S, H, D, n8 = 64, 4, 128, 64
    mixed = _bytes(n_slots=S, hv=H, hk=2, d=D, n8=n8)
    refit = _bytes(n_slots=S, hv=H, hk=2, d=D, n8=n8, fmt=stq.FMT_REFIT)
    # per-state column factors, squared row weights, accumulated impact
    assert refit == mixed + _r(S * H * D * 4) + _r(H * D * 4) + _r(H * D * 8)
    st = _fake_state(fmt=stq.FMT_REFIT, calibrated=1, n8=64, d=128)
    assert _decode(st) == E_ARG  # refit buffers missing
    for i, f in enumerate(("cs", "w2", "impact")):
        setattr(st, f, FAKE + 0x1000000 * (11 + i))
    st.calibrated = 0
    assert _decode(st) == E_STATE
    # row-impact calibration: REFIT only, flags RESET | FINALIZE, B >= 0
    st.calibrated = 1
    ci = lambda s_, B, flags, q=FAKE, dtype=0: lib.stq_calibrate_impact(  # noqa: E731
        ctypes.byref(s_), q, FAKE, dtype, FAKE, FAKE, B, flags, None)
    assert ci(st, -1, stq.CAL_RESET) == E_SHAPE
    assert ci(st, 2, stq.CAL_COLS) == E_ARG
    assert ci(st, 2, 0, q=None) == E_ARG
    assert ci(st, 2, 0, dtype=5) == E_ARG
    assert ci(st, 2, 0, dtype=stq.OUT_BF16) == E_ARG  # no readout here
    assert ci(st, 2, 0, q=FAKE + 2) == E_ARG
    mixed_st = _fake_state(calibrated=1)
    assert ci(mixed_st, 0, stq.CAL_RESET) == E_ARG


def test_gated_rejections():
    lib = stq.lib()
    src = _fake_state(calibrated=1)
    p = [FAKE] * 6

    def gated(a, b, gate=FAKE, B=2, dtype=0):
        return lib.stq_decode_step_gated(a, b, None, B, p[0], p[1], p[2], dtype, gate, p[4],
                                         p[5], None)

    assert gated(ctypes.byref(src), ctypes.byref(src), gate=None) == E_ARG
    assert gated(ctypes.byref(src), ctypes.byref(src), gate=FAKE + 2) == E_ARG
    assert gated(None, ctypes.byref(src)) == E_ARG
    assert gated(ctypes.byref(src), None) == E_ARG
    assert gated(ctypes.byref(src), ctypes.byref(src), B=0) == E_SHAPE
    assert gated(ctypes.byref(src), ctypes.byref(src), dtype=3) == E_ARG
    other = _fake_state(calibrated=1, n8=16)
    assert gated(ctypes.byref(src), ctypes.byref(other)) == E_SHAPE
    uncal = _fake_state(calibrated=0)
    assert gated(ctypes.byref(uncal), ctypes.byref(uncal)) == E_STATE
    # the scalar entry points still need alpha
    assert lib.stq_decode_step(ctypes.byref(src), None, 2, FAKE, FAKE, FAKE, 0, None, FAKE,
                               FAKE, None) == E_ARG
    # gated row-impact calibration: REFIT only, a gate whenever B > 0
    st = _fake_state(fmt=stq.FMT_REFIT, calibrated=1, n8=64, d=128)
    for i, f in enumerate(("cs", "w2", "impact")):
        setattr(st, f, FAKE + 0x1000000 * (11 + i))
    cg = lambda s_, B, flags, gate=FAKE: lib.stq_calibrate_impact_gated(  # noqa: E731
        ctypes.byref(s_), FAKE, FAKE, 0, gate, FAKE, B, flags, None)
    assert cg(st, 2, 0, gate=None) == E_ARG
    assert cg(st, 2, 0, gate=FAKE + 1) == E_ARG
    assert cg(st, -1, stq.CAL_RESET) == E_SHAPE
    assert cg(st, 2, stq.CAL_COLS) == E_ARG
    assert cg(_fake_state(calibrated=1), 0, stq.CAL_RESET) == E_ARG


def test_alloc_layout_arithmetic_and_rejections():
    S, H, D = 64, 32, 128
    for fmt in (stq.FMT_ALLOC, stq.FMT_ALLOC_REFIT):
        for nominal, piv in ((6, 26), (4, 0), (2, 100), (8, H * D)):
            slot = _alloc_slot_bytes(H, D, nominal, piv)
            expect = (_r(S * slot) + _r(S * H * D * 4) + _r(H * D * 4) * 2
                      + _r(H * D * 4) + _r(H * D * 8) + _r(H * 64 * D * 4) + _r(H * 64 * D * 8)
                      + _r(H * (8 + 64) * 4) + _r(H * D * 5 * 8) + _r(H * D * 8) + _r(H * 8))
            if fmt == stq.FMT_ALLOC_REFIT:
                expect += _r(S * H * D * 4) + _r(H * D * 4) + _r(H * D * 8)
            got = _bytes(n_slots=S, hv=H, hk=16, d=D, n8=0, fmt=fmt, nominal=nominal, piv=piv)
            assert got == expect, (fmt, nominal, piv)
    # the 6-bit budget with 0.625 % pivots: 12,288 B of codes per head plus
    # 256 B per pivot row (vs 96 B at 6 bits) and the padding allowance
    assert _alloc_slot_bytes(H, D, 6, 26) == 6 * (H * D - 26) * D // 8 + 2 * D * 26 + 16 * H
    for kw in (dict(n8=8), dict(nominal=5), dict(nominal=0), dict(piv=-1),
               dict(piv=4 * 64 + 1)):
        base = dict(n_slots=4, hv=4, hk=2, d=64, n8=0, fmt=stq.FMT_ALLOC, nominal=6, piv=0)
        base.update(kw)
        assert _bytes(**base) == 0, kw
    # other formats must leave the two fields at zero
    assert _bytes(n8=32, nominal=6) == 0
    assert _bytes(n8=32, piv=1) == 0


def _fake_alloc_state(fmt=stq.FMT_ALLOC, calibrated=1, d=64, hv=4, nominal=6, piv=3):
    st = stq.CState()
    st.desc = _desc(fmt=fmt, n8=0, d=d, hv=hv, nominal=nominal, piv=piv)
    for i, f in enumerate(("pool8", "r", "c", "perm", "colmax", "rowscore", "cal_colpart",
                           "cal_rowpart", "cs", "w2", "impact", "layout", "dist", "logret",
                           "nret")):
        setattr(st, f, FAKE + 0x1000000 * (i + 1))
    st.slot_bytes = _alloc_slot_bytes(hv, d, nominal, piv)
    st.calibrated = calibrated
    return st


def test_alloc_rejections():
    lib = stq.lib()
    st = _fake_alloc_state()
    assert _decode(_fake_alloc_state(calibrated=0)) == E_STATE
    bad = _fake_alloc_state()
    bad.slot_bytes += 16
    assert _decode(bad) == E_ARG  # slot_bytes must match the descriptor
    bad = _fake_alloc_state()
    bad.layout = None
    assert _decode(bad) == E_ARG
    # calibration flags: DIST only for ALLOC, ROWS not for ALLOC
    assert lib.stq_calibrate(ctypes.byref(st), FAKE, 1, stq.CAL_ROWS, None) == E_ARG
    assert lib.stq_calibrate(ctypes.byref(_fake_state(calibrated=1)), FAKE, 1, stq.CAL_DIST,
                             None) == E_ARG
    assert lib.stq_calibrate(ctypes.byref(st), None, 2, stq.CAL_DIST, None) == E_ARG
    assert lib.stq_set_calibration(ctypes.byref(st), FAKE, FAKE, None) == E_ARG
    # retention
    ret = lambda s_, a, g, B, f=0: lib.stq_calibrate_retention(  # noqa: E731
        ctypes.byref(s_), a, g, B, f, None)
    assert ret(st, FAKE, FAKE, 2) == E_ARG          # both gates
    assert ret(st, None, None, 2) == E_ARG          # neither
    assert ret(st, FAKE + 2, None, 2) == E_ARG      # misaligned
    assert ret(st, FAKE, None, -1) == E_SHAPE
    assert ret(st, FAKE, None, 2, stq.CAL_COLS) == E_ARG
    assert ret(_fake_state(calibrated=1), FAKE, None, 2) == E_ARG
    # assignment arguments
    assert lib.stq_allocate(ctypes.byref(st), 0, 0, None) == E_ARG       # horizon
    assert lib.stq_allocate(ctypes.byref(st), 64, 0x21, None) == E_ARG   # unknown class bit
    assert lib.stq_allocate(ctypes.byref(st), 64, 0x12, None) == E_ARG   # 6 bits not a candidate
    assert lib.stq_allocate(ctypes.byref(_fake_state(calibrated=1)), 64, 0, None) == E_ARG
    # installing a layout: counts on the host
    good = np.tile(np.array([0, 8, 24, 24, 8], np.int32), (4, 1))
    ok_counts = good.ctypes.data
    assert lib.stq_set_alloc_layout(ctypes.byref(st), None, FAKE, FAKE, None) == E_ARG
    assert lib.stq_set_alloc_layout(ctypes.byref(st), ok_counts, FAKE + 4, FAKE, None) == E_ARG
    short = good.copy()
    short[1, 4] -= 1                                  # head 1 sums to 63
    assert lib.stq_set_alloc_layout(ctypes.byref(st), short.ctypes.data, FAKE, FAKE,
                                    None) == E_ARG
    neg = good.copy()
    neg[0, 1], neg[0, 2] = -1, 25
    assert lib.stq_set_alloc_layout(ctypes.byref(st), neg.ctypes.data, FAKE, FAKE, None) == E_ARG
    fat = np.tile(np.array([64, 0, 0, 0, 0], np.int32), (4, 1))  # all pivots: too big
    assert lib.stq_set_alloc_layout(ctypes.byref(st), fat.ctypes.data, FAKE, FAKE,
                                    None) == E_SPACE


def test_calibrate_static_rejections():
    lib = stq.lib()
    big = stq.CState()
    big.desc = _desc(hv=128, hk=64, d=128, n8=64)  # 16384 head rows: over the fixed array
    assert lib.stq_calibrate_static(ctypes.byref(big), FAKE, 1, stq.CAL_COLS, None) == E_SPACE
    assert lib.stq_calibrate_static(None, FAKE, 1, stq.CAL_COLS, None) == E_ARG
    bad = stq.CState()
    bad.desc = _desc(hv=0)
    assert lib.stq_calibrate_static(ctypes.byref(bad), FAKE, 1, stq.CAL_COLS, None) == E_SHAPE
