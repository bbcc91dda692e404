"""stq_calibrate_static, the calibration entry point that allocates nothing
(its partial results live in a fixed per-GPU array of the library), against
stq_calibrate on the same records, through the C ABI: the folded statistics,
the column factors and the row order must be identical, bit for bit, on two
calls in a row, the second on a smaller state (fewer heads, smaller d_k,
fewer records) so that it runs over what the first left in the array.  Also
the ragged format, whose distortion pass follows the column pass."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from linear_attention_recurrent_rule_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from linear_attention_recurrent_rule_amd import stq  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

E_SPACE = 4


def _pair(geo):
    return stq.State(geo), stq.State(geo)


def _mixed_case(hv, hk, d, n8, n_rec, seed):
    print(f"[case] static calibration MIXED48 hv={hv} d={d} n8={n8} n_rec={n_rec}", flush=True)
    ref, got = _pair(stq.Geometry(2, hv, hk, d, n8, stq.FMT_MIXED48))
    rec = gu.dev(wl.random_states(n_rec, hv, d, seed=seed, outlier_sigma=1.0))
    for st, fn in ((ref, ref.calibrate), (got, got.calibrate_static)):
        fn(None, stq.CAL_RESET)
        fn(rec[: n_rec // 2], stq.CAL_COLS)
        fn(rec[n_rec // 2:], stq.CAL_COLS | stq.CAL_ROWS)
        fn(None, stq.CAL_FINALIZE)
    torch.cuda.synchronize()
    for name in ("colmax", "rowscore", "c", "perm"):
        a, b = getattr(ref, name), getattr(got, name)
        assert torch.equal(a, b), f"{name} differs"
    assert got.calibrated


def test_static_calibration_matches_two_calls_in_a_row():
    _mixed_case(32, 16, 128, 64, 6, seed=901)   # 4096 head rows
    _mixed_case(4, 2, 64, 16, 3, seed=902)      # smaller, over the first call's partials


def test_static_calibration_ragged_columns_and_distortion():
    hv, hk, d, n_rec = 4, 2, 64, 5
    print(f"[case] static calibration ALLOC hv={hv} d={d} n_rec={n_rec}", flush=True)
    geo = stq.Geometry(2, hv, hk, d, 0, stq.FMT_ALLOC, nominal_bits=6, n_pivot=3)
    ref, got = _pair(geo)
    rec = gu.dev(wl.random_states(n_rec, hv, d, seed=903, outlier_sigma=1.0))
    for st, fn in ((ref, ref.calibrate), (got, got.calibrate_static)):
        fn(None, stq.CAL_RESET)
        fn(rec, stq.CAL_COLS)
        fn(None, stq.CAL_FINALIZE)
        fn(rec, stq.CAL_DIST)
    torch.cuda.synchronize()
    for name in ("colmax", "c", "dist"):
        assert torch.equal(getattr(ref, name), getattr(got, name)), f"{name} differs"


def test_static_calibration_rejects_more_rows_than_the_array_holds():
    st = stq.State(stq.Geometry(1, 128, 64, 128, 64, stq.FMT_MIXED48))  # 16384 head rows
    rc = stq.lib().stq_calibrate_static(ctypes.byref(st.c_state), None, 0, stq.CAL_RESET, None)
    assert rc == E_SPACE
    np.testing.assert_array_equal(st.colmax.cpu().numpy(), 0)  # nothing queued
