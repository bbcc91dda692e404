"""Pools larger than 4 GiB: decode steps on the highest slots of a state
sized for 20,000 sequences of 32 value heads at d = 128 (about 8.2 GB for the
6-bit mix, 8.6 GB for the ragged format), so every byte offset of the touched
rows exceeds 32 bits.  Sampled against the oracle; the untouched slots below
stay untouched."""
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
from tests.test_gpu_alloc import _compare, pivot_allowance  # noqa: E402

N_SLOTS, HV, HK, D = 20000, 32, 16, 128
B = 8


def _top_slots():
    return np.arange(N_SLOTS - B, N_SLOTS, dtype=np.int32)[::-1].copy()  # reversed order


def test_mixed_top_slots_of_a_large_pool(oracle_mod):
    n8 = 64
    print(f"[case] mixed pool of {N_SLOTS} slots, slots {N_SLOTS - B}..{N_SLOTS - 1}", flush=True)
    st = gu.make_state(B, HV, HK, D, n8, n_slots=N_SLOTS)
    assert (N_SLOTS - B) * HV * n8 * D > 1 << 32  # offsets of the touched rows
    ps = wl.random_packed_state(B, HV, D, n8, seed=61)
    slots = _top_slots()
    gu.load_packed(st, ps, slots=slots)
    x = wl.draw_inputs(B, HK, HV, D, dtype="bf16", seed=61, step=0)
    o = gu.gpu_step(st, x, slots_t=gu.dev(slots))
    p8, p4, r = gu.read_packed(st, slots=slots)
    ref = gu.oracle_step_on(oracle_mod, ps, x, nthreads=16)
    print(gu.compare_step(dict(pool8=p8, pool4=p4, r=r, o=o), ref, n8=n8, d=D, label="top slots"))
    # a slot just below the touched range still holds the initial state
    below = np.array([N_SLOTS - B - 1, 0], np.int32)
    q8, q4, rq = gu.read_packed(st, slots=below)
    assert not q8.any() and not q4.any()
    assert np.all(rq == np.float32(2.0 ** -126))
    del st
    torch.cuda.empty_cache()


def test_ragged_top_slots_of_a_large_pool(oracle_mod):
    print(f"[case] ragged pool of {N_SLOTS} slots", flush=True)
    counts = wl.calibration_shaped_counts(HV, D, seed=62, two_bit_heads=2)
    g = wl.rng_for(62, 1)
    perm = np.stack([g.permutation(D) for _ in range(HV)]).astype(np.int32)
    c = g.lognormal(0.0, 0.7, size=(HV, D)).astype(np.float32)
    st = stq.State(stq.Geometry(N_SLOTS, HV, HK, D, 0, stq.FMT_ALLOC, nominal_bits=8,
                                n_pivot=int(counts[:, 0].sum())))
    assert (N_SLOTS - B) * st.slot_bytes > 1 << 32
    st.set_alloc_layout(counts, gu.dev(c), gu.dev(perm))
    pool, r = wl.random_ragged_state(B, counts, D, st.slot_bytes, seed=63)
    slots = _top_slots()
    idx = torch.from_numpy(slots.astype(np.int64)).cuda()
    st.pool[idx] = gu.dev(pool)
    st.r[idx] = gu.dev(r)
    x = wl.draw_inputs(B, HK, HV, D, dtype="bf16", seed=63, step=0)
    q, k, v, a, b = gu.inputs_to_device(x)
    o = st.decode_step(q, k, v, a, b, slots=gu.dev(slots))
    torch.cuda.synchronize()
    gp, gr = st.pool[idx].cpu().numpy(), st.r[idx].cpu().numpy()
    ref = oracle_mod.alloc_step(pool, r, counts, perm, x.q, x.k, x.v, x.alpha, x.beta, c=c,
                                nthreads=16, want_X=True)
    print(_compare(gp, gr, ref["pool"], ref["r"], counts, D, "ragged top slots",
                   o=o.cpu().numpy(), ref_o=ref["o"],
                   pivot_err=pivot_allowance(pool, r, counts, perm, c, x.k, x.v, x.beta, ref["X"], D,
                                             alpha=x.alpha)))
    assert not st.pool[N_SLOTS - B - 1].any().item()
    del st
    torch.cuda.empty_cache()
