"""The Python binding checks every tensor it hands to the C ABI - dtype, exact
shape, device, contiguity, byte sizes - and raises ValueError before anything
is queued.  Host-only: the state here is a binding object over no device
memory (its device is the meta device), and every call below must fail in
the binding's own checks, so nothing reaches the library."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
stq = pytest.importorskip("linear_attention_recurrent_rule_amd.stq")

B, HV, HK, D = 3, 4, 2, 64


def _state(fmt=stq.FMT_MIXED48, n8=32, nominal=0, piv=0):
    st = stq.State.__new__(stq.State)
    st.geo = stq.Geometry(8, HV, HK, D, n8, fmt, nominal, piv)
    st.buffer = torch.empty(0, dtype=torch.uint8, device="meta")
    st._device = st.buffer.device  # as State.__init__ sets it
    return st


def _t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _step_args(**over):
    a = dict(q=_t(B, HK, D), k=_t(B, HK, D), v=_t(B, HV, D), alpha=_t(B, HV), beta=_t(B, HV))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(q=_t(B, HK + 1, D)), "q must have shape"),
    (dict(k=_t(B, HK, D + 1)), "k must have shape"),
    (dict(v=_t(B, HK, D)), "v must have shape"),
    (dict(alpha=_t(B, HV, 1)), "alpha must have shape"),
    (dict(beta=_t(B + 1, HV)), "beta must have shape"),
    (dict(alpha=_t(B, HV, dtype=torch.float64)), "alpha must be float32"),
    (dict(q=_t(B, HK, D, dtype=torch.float16), k=_t(B, HK, D, dtype=torch.float16),
          v=_t(B, HV, D, dtype=torch.float16)), "float32 or bfloat16"),
    (dict(v=_t(B, HV, D, dtype=torch.bfloat16)), "share one dtype"),
    (dict(beta=None), "beta is required"),
    (dict(q=np.zeros((B, HK, D), np.float32)), "torch tensor"),
    ({}, "must be a device tensor"),
])
def test_decode_step_checks(over, msg):
    st = _state()
    with pytest.raises(ValueError, match=msg):
        st.decode_step(**_step_args(**over))


def test_decode_readout_slots_and_gate_checks():
    st = _state()
    a = _step_args()
    with pytest.raises(ValueError, match="o must have shape"):
        st.decode_step(**a, o=_t(B, HV, D + 2))
    with pytest.raises(ValueError, match="o must be a float32 or bfloat16"):
        st.decode_step(**a, o=_t(B, HV, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="slots must be int32"):
        st.decode_step(**a, slots=_t(B, dtype=torch.int64))
    with pytest.raises(ValueError, match="slots must have shape"):
        st.decode_step(**a, slots=_t(B + 1, dtype=torch.int32))
    g = dict(q=a["q"], k=a["k"], v=a["v"], beta=a["beta"])
    with pytest.raises(ValueError, match="gate must have shape"):
        st.decode_step_gated(**g, gate=_t(B, HV))
    with pytest.raises(ValueError, match="gate is required"):
        st.decode_step_gated(**g, gate=None)
    with pytest.raises(ValueError, match="alpha must have shape"):
        st.decode_step_into(_state(), **_step_args(alpha=_t(B)))


def test_pack_dequant_calibrate_checks():
    st = _state()
    with pytest.raises(ValueError, match="S must have shape"):
        st.pack(_t(B, HV, D, D + 1))
    with pytest.raises(ValueError, match="S must be float32"):
        st.pack(_t(B, HV, D, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="slots must have shape"):
        st.pack(_t(B, HV, D, D), slots=_t(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="S must be a device tensor"):
        st.pack(_t(B, HV, D, D))
    with pytest.raises(ValueError, match="out must have shape"):
        st.dequant(B=2, out=_t(3, HV, D, D))
    with pytest.raises(ValueError, match="records must have shape"):
        st.calibrate(_t(2, HV, D, D - 1), stq.CAL_COLS)
    with pytest.raises(ValueError, match="records must be float32"):
        st.calibrate(_t(2, HV, D, D, dtype=torch.float64), stq.CAL_COLS)
    with pytest.raises(ValueError, match="c must have shape"):
        st.set_calibration(_t(HV, D + 1), _t(HV, D, dtype=torch.int32))
    with pytest.raises(ValueError, match="perm must be int32"):
        st.set_calibration(_t(HV, D), _t(HV, D, dtype=torch.int64))


def test_impact_retention_layout_checks():
    st = _state(fmt=stq.FMT_REFIT)
    q, k = _t(B, HK, D), _t(B, HK, D)
    with pytest.raises(ValueError, match="beta must have shape"):
        st.calibrate_impact(q, k, _t(B, HV), _t(B, HV + 1), 0)
    with pytest.raises(ValueError, match="share one dtype"):
        st.calibrate_impact(q, _t(B, HK, D, dtype=torch.bfloat16), _t(B, HV), _t(B, HV), 0)
    with pytest.raises(ValueError, match="gate must have shape"):
        st.calibrate_impact(q, k, None, _t(B, HV), 0, gate=_t(B, HV))
    al = _state(fmt=stq.FMT_ALLOC, n8=0, nominal=6, piv=2)
    with pytest.raises(ValueError, match="alpha must have shape"):
        al.calibrate_retention(alpha=_t(B, HV, D))
    with pytest.raises(ValueError, match="gate must have shape"):
        al.calibrate_retention(gate=_t(B, HV))
    with pytest.raises(ValueError, match="counts must have shape"):
        al.set_alloc_layout(np.zeros((HV, 4), np.int32), _t(HV, D), _t(HV, D, dtype=torch.int32))
    with pytest.raises(ValueError, match="perm must have shape"):
        al.set_alloc_layout(np.zeros((HV, 5), np.int32), _t(HV, D), _t(HV, D + 1,
                                                                       dtype=torch.int32))


def test_stream_copy_checks():
    with pytest.raises(ValueError, match="src must be a device tensor"):
        stq.stream_copy(_t(16), _t(16))
    with pytest.raises(ValueError, match="src must be a torch tensor"):
        stq.stream_copy(np.zeros(4), _t(4))
