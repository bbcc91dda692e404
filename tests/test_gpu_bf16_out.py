"""The bf16 readout (STQ_OUT_BF16): every decode kernel, given the same state
and inputs, writes the same packed state as with an fp32 readout, and each
bf16 readout element is the fp32 readout rounded to nearest even (NaN where
the slot is skipped).  The fp32 readout itself is held to the oracle by the
other parity tests, so the bf16 one is within half a bf16 ulp of a value that
passed them.  Bit-exact bar: both sides round the same fp32 number."""
from __future__ import annotations

import numpy as np
import pytest

from linear_attention_recurrent_rule_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from linear_attention_recurrent_rule_amd import stq  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

B, HV, HK = 37, 4, 2


def _slots():
    s = np.arange(B, dtype=np.int32)
    s[5] = -1  # skipped: its readout is NaN
    return gu.dev(s)


def _check_readout(o32, o16):
    assert o16.dtype == torch.bfloat16 and o16.shape == o32.shape
    want = o32.to(torch.bfloat16)
    nan32, nan16 = torch.isnan(o32), torch.isnan(o16)
    assert torch.equal(nan32, nan16)
    assert nan32[5].all() and not nan32[torch.arange(B) != 5].any()
    ok = ~nan32
    assert torch.equal(o16.view(torch.int16)[ok], want.view(torch.int16)[ok])


def _state_tensors(st):
    return [t for t in (st.pool8, st.pool4, st.r, st.pool, st.cs) if t is not None]


def _same_state(a, b):
    torch.cuda.synchronize()
    for x, y in zip(_state_tensors(a), _state_tensors(b)):
        assert torch.equal(x, y)


def _run_pair(make, x, gate=None):
    """Two identical states, one step each: fp32 readout, then bf16."""
    s32, s16 = make(), make()
    q, k, v, a, b = gu.inputs_to_device(x)
    slots = _slots()
    if gate is None:
        o32 = s32.decode_step(q, k, v, a, b, slots=slots)
        o16 = s16.decode_step(q, k, v, a, b, slots=slots, o_dtype=torch.bfloat16)
    else:
        g = gu.dev(gate)
        o32 = s32.decode_step_gated(q, k, v, g, b, slots=slots)
        o16 = s16.decode_step_gated(q, k, v, g, b, slots=slots, o_dtype=torch.bfloat16)
    _same_state(s32, s16)
    _check_readout(o32, o16)


@pytest.mark.parametrize("d,n8,dtype,gated", [(128, 64, "bf16", False), (128, 40, "bf16", False),
                                               (128, 64, "f32", True), (64, 32, "bf16", False),
                                               (32, 8, "f32", True)])
def test_bf16_readout_mixed(d, n8, dtype, gated):
    """d = 128 at n8 = 64 takes a compile-time instance of the matrix-core
    kernel, n8 = 40 the one that reads the split at run time; d = 64 and 32
    take the generic kernel."""
    print(f"[case] mixed d={d} n8={n8} {dtype} gated={gated}", flush=True)
    ps = wl.random_packed_state(B, HV, d, n8, seed=700 + d + n8)
    x = wl.draw_inputs(B, HK, HV, d, dtype=dtype, seed=701, step=0)
    gate = wl.draw_gate(B, HV, d, seed=702, step=0) if gated else None

    def make():
        st = gu.make_state(B, HV, HK, d, n8)
        gu.load_packed(st, ps)
        return st

    _run_pair(make, x, gate)


@pytest.mark.parametrize("fmt", ["int8row", "fp32", "refit"])
def test_bf16_readout_other_formats(fmt):
    d = 128 if fmt != "fp32" else 64
    print(f"[case] {fmt} d={d}", flush=True)
    x = wl.draw_inputs(B, HK, HV, d, dtype="bf16", seed=711, step=0)
    g = wl.rng_for(712, d)
    if fmt == "int8row":
        ps = wl.random_packed_state(B, HV, d, d, seed=713, c_one=True, identity_perm=True)

        def make():
            st = gu.make_state(B, HV, HK, d, d, fmt=stq.FMT_INT8ROW)
            gu.load_packed(st, ps)
            return st
    elif fmt == "fp32":
        S = gu.dev(g.standard_normal((B, HV, d, d), dtype=np.float32))

        def make():
            st = gu.make_state(B, HV, HK, d, 0, fmt=stq.FMT_FP32)
            st.pack(S)
            return st
    else:
        n8 = 64
        ps = wl.random_packed_state(B, HV, d, n8, seed=714, full_rows=True)
        cs = g.lognormal(0.0, 0.7, size=(B, HV, d)).astype(np.float32)
        w2 = (g.uniform(0.05, 1.0, size=(HV, d)) ** 0.5).astype(np.float32)

        def make():
            st = gu.make_state(B, HV, HK, d, n8, fmt=stq.FMT_REFIT)
            st.set_calibration(gu.dev(ps.c), gu.dev(ps.perm))
            st.pool8.copy_(gu.dev(ps.pool8))
            st.pool4.copy_(gu.dev(ps.pool4))
            st.r.copy_(gu.dev(ps.r))
            st.cs.copy_(gu.dev(cs))
            st.w2.copy_(gu.dev(w2))
            return st

    _run_pair(make, x)


@pytest.mark.parametrize("d,gated", [(128, False), (128, True), (64, False)])
def test_bf16_readout_ragged(d, gated):
    """d = 128 takes the ragged matrix-core kernel, d = 64 the generic one."""
    print(f"[case] ragged d={d} gated={gated}", flush=True)
    counts = wl.calibration_shaped_counts(HV, d, seed=720 + d, two_bit_heads=1)
    g = wl.rng_for(721, d)
    perm = np.stack([g.permutation(d) for _ in range(HV)]).astype(np.int32)
    c = g.lognormal(0.0, 0.7, size=(HV, d)).astype(np.float32)
    x = wl.draw_inputs(B, HK, HV, d, dtype="bf16", seed=722, step=0)
    gate = wl.draw_gate(B, HV, d, seed=723, step=0) if gated else None
    holder = {}

    def make():
        st = stq.State(stq.Geometry(B, HV, HK, d, 0, stq.FMT_ALLOC, nominal_bits=8,
                                    n_pivot=int(counts[:, 0].sum())))
        st.set_alloc_layout(counts, gu.dev(c), gu.dev(perm))
        if "pool" not in holder:
            holder["pool"], holder["r"] = wl.random_ragged_state(B, counts, d, st.slot_bytes,
                                                                 seed=724)
        st.pool.copy_(gu.dev(holder["pool"]))
        st.r.copy_(gu.dev(holder["r"]))
        return st

    _run_pair(make, x, gate)


def test_bf16_readout_fullsize():
    """The launch the benchmark times for this variant: B = 1024 sequences, 32
    value heads over 16 key heads, d = 128, the 6-bit mix, bf16 inputs."""
    w = wl.WORKLOADS["highconc_6bit"]
    print(f"[case] bf16 readout full size B={w.B} hv={w.hv} hk={w.hk} d={w.d} n8={w.n8}",
          flush=True)
    ps = wl.random_packed_state(w.B, w.hv, w.d, w.n8, seed=w.seed + 740)
    x = wl.workload_inputs(w, 0)
    q, k, v, a, b = gu.inputs_to_device(x)
    s32 = gu.make_state(w.B, w.hv, w.hk, w.d, w.n8)
    gu.load_packed(s32, ps)
    s16 = gu.make_state(w.B, w.hv, w.hk, w.d, w.n8)
    gu.load_packed(s16, ps)
    o32 = s32.decode_step(q, k, v, a, b)
    o16 = s16.decode_step(q, k, v, a, b, o_dtype=torch.bfloat16)
    _same_state(s32, s16)
    assert o16.dtype == torch.bfloat16 and o16.shape == o32.shape
    assert not torch.isnan(o32).any()
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))


def test_bf16_readout_rejects_other_dtypes():
    st = gu.make_state(2, HV, HK, 32, 8)
    ps = wl.random_packed_state(2, HV, 32, 8, seed=730)
    gu.load_packed(st, ps)
    x = wl.draw_inputs(2, HK, HV, 32, dtype="f32", seed=731, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    with pytest.raises(ValueError):
        st.decode_step(q, k, v, a, b, o_dtype=torch.float16)
