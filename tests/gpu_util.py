"""Helpers shared by the GPU tests: move seeded host workloads to the device,
run the HIP path through the C ABI binding, and compare with the oracle to the
parity bar (codes >= 99.99 % identical and the rest within +-1, row factors
within 1e-6 relative, readout within 1e-4 relative L2)."""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_recurrent_rule_amd import stq
from linear_attention_recurrent_rule_amd import workloads as wl

CODE_MATCH_MIN = 0.9999
R_RTOL = 1e-6
O_REL_L2 = 1e-4


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def inputs_to_device(x: wl.StepInputs):
    if x.dtype == "bf16":
        conv = lambda bits: dev(bits.view(np.int16)).view(torch.bfloat16)  # noqa: E731
        q, k, v = conv(x.q_bits), conv(x.k_bits), conv(x.v_bits)
    else:
        q, k, v = dev(x.q), dev(x.k), dev(x.v)
    return q, k, v, dev(x.alpha), dev(x.beta)


def make_state(B, hv, hk, d, n8, fmt=stq.FMT_MIXED48, n_slots=None):
    return stq.State(stq.Geometry(n_slots or B, hv, hk, d, n8, fmt))


def load_packed(st: stq.State, ps: wl.PackedState, slots: np.ndarray | None = None):
    """Install a host-generated packed state (and its calibration) into st."""
    if st.geo.fmt == stq.FMT_MIXED48:
        st.set_calibration(dev(ps.c), dev(ps.perm))
    idx = slice(None) if slots is None else torch.from_numpy(slots.astype(np.int64)).cuda()
    if st.pool8 is not None and ps.pool8.size:
        st.pool8[idx] = dev(ps.pool8)
    if st.pool4 is not None and ps.pool4.size:
        st.pool4[idx] = dev(ps.pool4)
    st.r[idx] = dev(ps.r)
    torch.cuda.synchronize()


def read_packed(st: stq.State, slots: np.ndarray | None = None):
    idx = slice(None) if slots is None else torch.from_numpy(slots.astype(np.int64)).cuda()
    torch.cuda.synchronize()
    g = st.geo
    r = st.r[idx].cpu().numpy()
    B = r.shape[0]
    p8 = (st.pool8[idx].cpu().numpy() if st.pool8 is not None
          else np.zeros((B, g.n_heads_v, 0, g.d), np.int8))
    p4 = (st.pool4[idx].cpu().numpy() if st.pool4 is not None
          else np.zeros((B, g.n_heads_v, 0, g.d // 2), np.uint8))
    return p8, p4, r


def _empty8(B, hv, d):
    return np.zeros((B, hv, 0, d), np.int8)


# With the oracle's exact code values at hand, a code may differ from the
# oracle's only where that value lies this close to a rounding boundary: the
# kernel evaluates it in fp32 (|t| <= 127, a few roundings and a 1-ulp
# reciprocal), well within 32 ulps of |t|.
TIE_WINDOW = 2.0 ** -12


def exact_code_values(X, r, c, perm):
    """t = X / (r' c) per stored code, physical rows [B][Hv][d][d]: X the
    oracle's updated state (logical rows), r the new row factors (physical
    rows), c the column factors per head [Hv][d] or per state [B][Hv][d]."""
    B, hv = r.shape[:2]
    Xp = np.take_along_axis(X, perm[None, :, :, None], axis=2)
    cc = c.astype(np.float64)
    cc = cc[None, :, None, :] if cc.ndim == 2 else cc[:, :, None, :]
    return Xp / (r.astype(np.float64)[..., None] * cc)


def compare_step(gpu: dict, ref: dict, *, n8: int, d: int, label: str = "",
                 t_exact=None) -> dict:
    """Per-step parity against the oracle; returns statistics, raises on failure.
    With t_exact (exact_code_values of the oracle's step), every code that
    differs must sit within TIE_WINDOW of a rounding boundary, in place of
    the bar on the share of identical codes (for inputs whose values cluster
    at ties)."""
    B, hv = ref["r"].shape[:2]
    g8 = gpu["pool8"] if gpu["pool8"] is not None else _empty8(B, hv, d)
    g4 = gpu["pool4"] if gpu["pool4"] is not None else np.zeros((B, hv, 0, d // 2), np.uint8)
    zg = wl.unpack_codes(g8.reshape(B, hv, n8, d), g4.reshape(B, hv, d - n8, d // 2)).astype(np.int32)
    zr = wl.unpack_codes(ref["pool8"], ref["pool4"]).astype(np.int32)
    diff = np.abs(zg - zr)
    match = float(np.mean(diff == 0))
    max_code = int(diff.max()) if diff.size else 0
    rr = np.abs(gpu["r"].astype(np.float64) - ref["r"]) / np.abs(ref["r"].astype(np.float64))
    max_r = float(rr.max())
    og = gpu["o"].astype(np.float64)
    orf = ref["o"].astype(np.float64)
    num = np.sqrt(np.sum((og - orf) ** 2, axis=-1))
    den = np.sqrt(np.sum(orf ** 2, axis=-1))
    rel_o = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    max_o = float(rel_o.max())
    stats = dict(code_match=match, max_code_diff=max_code, max_r_rel=max_r, max_o_rel_l2=max_o,
                 n_codes=int(diff.size))
    assert np.all(np.isfinite(gpu["o"])), f"{label}: non-finite readout"
    if t_exact is None:
        assert match >= CODE_MATCH_MIN, f"{label}: codes identical {match:.6f} < {CODE_MATCH_MIN} {stats}"
    else:
        t = t_exact[diff != 0]
        off = np.abs(t - np.floor(t) - 0.5) if t.size else np.zeros(1)
        stats["max_tie_offset"] = float(off.max())
        assert off.max() <= TIE_WINDOW, f"{label}: a code differs away from a tie {stats}"
    assert max_code <= 1, f"{label}: code differs by {max_code} {stats}"
    assert max_r <= R_RTOL, f"{label}: row factor rel diff {max_r:.3g} {stats}"
    assert max_o <= O_REL_L2, f"{label}: readout rel L2 {max_o:.3g} {stats}"
    return stats


def gpu_step(st: stq.State, x: wl.StepInputs, slots_t=None):
    q, k, v, a, b = inputs_to_device(x)
    o = st.decode_step(q, k, v, a, b, slots=slots_t)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def oracle_step_on(oracle_mod, ps: wl.PackedState, x: wl.StepInputs, nthreads: int = 8):
    return oracle_mod.step(ps.pool8, ps.pool4, ps.r, ps.c, ps.perm, x.q, x.k, x.v, x.alpha,
                           x.beta, n8=ps.n8, nthreads=nthreads)
