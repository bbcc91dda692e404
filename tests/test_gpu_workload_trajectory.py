"""Per-step parity along the GPU's own trajectory of the serving and the
high-concurrency workloads (B = 256 and 1024 sequences, 32 value heads over
16 key heads, d = 128, bf16 inputs, the 6-bit mix and, at B = 1024, the
4.5-bit mix of 16 int8 rows), in the launch
configuration the benchmark times.  The library generates nothing here: S0
and the inputs come from the seeded generators, the library calibrates from
32 unquantized steps, packs S0 and runs the workload's T = 100 steps in
place; at steps 1, 2, T/2 and T the oracle repeats the step on every unit
from the state the GPU held before it, and the GPU's result must match it to
the parity bar (codes >= 99.99 % identical and the rest +-1, row factors
within 1e-6 relative, readout within 1e-4 relative L2).  Per-step rather
than end-to-end, because a code may legitimately flip by one at a rounding
tie and the two trajectories then differ by that code.  One layer of the
stacked workload runs its 2048 steps with inputs drawn on the device and is
checked every 256th step on 1/16 of its sequences."""
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


def _calibrate(w, S0_dev):
    """c and perm from the workload's calibration stream (32 unquantized
    steps on the FP32-state kernel, column maxima over all of them, row
    scores from the last)."""
    fp = gu.make_state(w.B, w.hv, w.hk, w.d, 0, fmt=stq.FMT_FP32)
    fp.pack(S0_dev)
    cal = gu.make_state(1, w.hv, w.hk, w.d, w.n8)
    cal.calibrate(None, stq.CAL_RESET)
    for t in range(w.calib_steps):
        q, k, v, a, b = gu.inputs_to_device(wl.workload_inputs(w, t, calibration=True))
        fp.decode_step(q, k, v, a, b)
        last = t == w.calib_steps - 1
        cal.calibrate(fp.s32, stq.CAL_COLS | (stq.CAL_ROWS if last else 0))
    cal.calibrate(None, stq.CAL_FINALIZE)
    torch.cuda.synchronize()
    return cal.c.clone(), cal.perm.clone()


@pytest.mark.parametrize("name", ["serving_6bit", "highconc_6bit", "highconc_4p5bit"])
def test_workload_trajectory_checkpoints(oracle_mod, name):
    w = wl.WORKLOADS[name]
    checks = {1, 2, w.T // 2, w.T}
    print(f"[case] {name}: B={w.B} hv={w.hv} hk={w.hk} d={w.d} n8={w.n8} T={w.T}, "
          f"checked steps {sorted(checks)}", flush=True)
    S0 = gu.dev(wl.initial_state(w))
    c, perm = _calibrate(w, S0)
    st = gu.make_state(w.B, w.hv, w.hk, w.d, w.n8)
    st.set_calibration(c, perm)
    st.pack(S0)
    del S0
    torch.cuda.empty_cache()
    c_h, perm_h = c.cpu().numpy(), perm.cpu().numpy()
    for t in range(w.T):
        x = wl.workload_inputs(w, t)
        if t + 1 not in checks:
            gu.gpu_step(st, x)
            continue
        p8, p4, r = gu.read_packed(st)
        o = gu.gpu_step(st, x)
        gp8, gp4, gr = gu.read_packed(st)
        ref = gu.oracle_step_on(oracle_mod, wl.PackedState(p8, p4, r, c_h, perm_h, w.n8), x,
                                nthreads=16)
        stats = gu.compare_step(dict(pool8=gp8, pool4=gp4, r=gr, o=o), ref, n8=w.n8, d=w.d,
                                label=f"{name} step {t + 1}")
        print(f"{name} step {t + 1}: {stats}", flush=True)
        del p8, p4, r, gp8, gp4, gr, ref


def _device_inputs(w, t):
    """One step of the workload's laws drawn on the device (q, k ~ N(0, 1)
    L2-normalised, v ~ N(0, 1), alpha ~ U(lo, 1), beta = sigmoid(N(0, 1)),
    bf16 by round-to-nearest-even): 2048 host draws would take minutes."""
    g = torch.Generator(device="cuda").manual_seed(w.seed * 1_000_003 + t)
    B, hk, hv, d = w.B, w.hk, w.hv, w.d
    q = torch.randn(B, hk, d, device="cuda", generator=g)
    k = torch.randn(B, hk, d, device="cuda", generator=g)
    q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16).contiguous()
    k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16).contiguous()
    v = torch.randn(B, hv, d, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    a = (torch.rand(B, hv, device="cuda", generator=g) * (1.0 - w.alpha_lo) + w.alpha_lo).contiguous()
    b = torch.sigmoid(torch.randn(B, hv, device="cuda", generator=g)).contiguous()
    return q, k, v, a, b


def test_stacked_layer_long_trajectory(oracle_mod):
    """One layer of the stacked workload (B = 512) over its T = 2048 steps;
    at every 256th step the oracle repeats the step on 1/16 of the
    sequences (all heads of each) from the GPU's state before it."""
    w = wl.WORKLOADS["stacked_6bit"]
    checks = set(range(256, w.T + 1, 256))
    bs = np.sort(wl.rng_for(w.seed, 78).choice(w.B, w.B // 16, replace=False)).astype(np.int32)
    print(f"[case] stacked_6bit layer 0: B={w.B} T={w.T}, sequences {bs[:4].tolist()}..., "
          f"checked every 256th step", flush=True)
    S0 = gu.dev(wl.initial_state(w))
    c, perm = _calibrate(w, S0)
    st = gu.make_state(w.B, w.hv, w.hk, w.d, w.n8)
    st.set_calibration(c, perm)
    st.pack(S0)
    del S0
    torch.cuda.empty_cache()
    c_h, perm_h = c.cpu().numpy(), perm.cpu().numpy()
    idx = torch.from_numpy(bs.astype(np.int64)).cuda()
    for t in range(w.T):
        q, k, v, a, b = _device_inputs(w, t)
        if t + 1 not in checks:
            st.decode_step(q, k, v, a, b)
            continue
        p8, p4, r = gu.read_packed(st, slots=bs)
        o = st.decode_step(q, k, v, a, b)
        gp8, gp4, gr = gu.read_packed(st, slots=bs)
        host = lambda x_: x_[idx].float().cpu().numpy()  # noqa: E731
        x = wl.StepInputs(host(q), host(k), host(v), host(a), host(b), "bf16")
        ref = gu.oracle_step_on(oracle_mod, wl.PackedState(p8, p4, r, c_h, perm_h, w.n8), x,
                                nthreads=16)
        stats = gu.compare_step(dict(pool8=gp8, pool4=gp4, r=gr, o=host(o)), ref, n8=w.n8,
                                d=w.d, label=f"stacked step {t + 1}")
        print(f"stacked step {t + 1}: {stats}", flush=True)
