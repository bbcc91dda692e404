"""Seeded synthetic workloads for the quantized gated delta-rule decode step.

This module only draws random numbers and arranges them into arrays: it holds
none of the decode step's arithmetic (no update, no readout, no quantization).
Both the CPU oracle and the GPU path consume what it produces.

The pages measure on real hybrid models (Qwen3.8-27B GDN heads and Kimi-Linear
KDA heads, 128 x 128 states, served at batch sizes up to 512; STEPQuant paper,
Sec. 5.1 and App. F.5) and public suites; none of those are available here.
These generators stand in for them with the same state shape and the row and
column outlier structure the paper reports for recurrent states (Sec. 4.2,
App. B.6: max-to-median RMS contrasts of about 10x along key rows and 19x
along value columns).

Laws (per sequence b, head h, step t):
  q, k ~ N(0, 1)^d, then L2-normalised in fp32     (key head)
  v    ~ N(0, 1)^d                                  (value head)
  alpha ~ U(lo, 1),  beta = sigmoid(N(0, 1))        (value head)
  bf16 inputs are the fp32 draws rounded to nearest-even bf16.
Per-key-row gates of the KDA form (draw_gate; one fp32 per sequence, value
head and logical key row, from a stream of its own):
  d_i = sigmoid(N(2.5, 1.5))   (median 0.92; about 5 % of rows below 0.5)
Random packed states (for per-step parity from an arbitrary state) draw codes
uniformly from the symmetric range of their row width, log-uniform row factors,
log-normal column factors and a random physical row order per head.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------- configs --


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    hk: int
    hv: int
    d: int
    n8: int
    T: int
    dtype: str  # "f32" or "bf16" for q, k, v
    seed: int
    calib_seed: int | None
    s0: str  # "zero", "normal", "outlier"
    s0_scale: float = 1.0  # std of the normal part
    outlier_sigma: float = 0.0  # log-normal sigma of row/column factors
    alpha_lo: float = 0.9
    layers: int = 1
    calib_steps: int = 32
    extra: dict = field(default_factory=dict)

    @property
    def units(self) -> int:
        return self.B * self.hv


WORKLOADS = {
    "tiny": Workload("tiny", B=1, hk=1, hv=1, d=16, n8=16, T=64, dtype="f32", seed=0,
                     calib_seed=None, s0="zero"),
    "small_mixed": Workload("small_mixed", B=8, hk=4, hv=4, d=64, n8=32, T=256, dtype="f32",
                            seed=1, calib_seed=1001, s0="normal", s0_scale=0.1),
    "serving_6bit": Workload("serving_6bit", B=256, hk=16, hv=32, d=128, n8=64, T=100,
                             dtype="bf16", seed=2, calib_seed=1002, s0="outlier",
                             outlier_sigma=1.0),
    "highconc_4p5bit": Workload("highconc_4p5bit", B=1024, hk=16, hv=32, d=128, n8=16, T=100,
                                dtype="bf16", seed=3, calib_seed=1003, s0="outlier",
                                outlier_sigma=1.5),
    "highconc_6bit": Workload("highconc_6bit", B=1024, hk=16, hv=32, d=128, n8=64, T=100,
                              dtype="bf16", seed=3, calib_seed=1003, s0="outlier",
                              outlier_sigma=1.5),
    "stacked_6bit": Workload("stacked_6bit", B=512, hk=16, hv=32, d=128, n8=64, T=2048,
                             dtype="bf16", seed=4, calib_seed=1004, s0="outlier",
                             outlier_sigma=1.0, alpha_lo=0.95, layers=48),
}

# stream tags keep the random streams of different purposes independent
_TAG_INPUTS = 11
_TAG_S0 = 12
_TAG_PACKED = 13
_TAG_RECORDS = 14
_TAG_GATE = 15


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))


# -------------------------------------------------------------- bf16 utils --


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ inputs --


@dataclass
class StepInputs:
    """One decode step's inputs.  q, k, v are fp32 arrays holding exactly the
    values the kernel sees (bf16-representable when dtype == 'bf16');
    q_bits, k_bits, v_bits hold the bf16 patterns in that case."""
    q: np.ndarray  # [B][Hk][d]
    k: np.ndarray  # [B][Hk][d]
    v: np.ndarray  # [B][Hv][d]
    alpha: np.ndarray  # [B][Hv]
    beta: np.ndarray  # [B][Hv]
    dtype: str
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x / n).astype(np.float32)


def draw_inputs(B: int, hk: int, hv: int, d: int, *, dtype: str, seed: int, step: int,
                alpha_lo: float = 0.9, stream: int = _TAG_INPUTS, layer: int = 0) -> StepInputs:
    g = rng_for(seed, stream, layer, step)
    q = _l2n(g.standard_normal((B, hk, d), dtype=np.float32))
    k = _l2n(g.standard_normal((B, hk, d), dtype=np.float32))
    v = g.standard_normal((B, hv, d), dtype=np.float32)
    alpha = g.uniform(alpha_lo, 1.0, size=(B, hv)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-g.standard_normal((B, hv))))).astype(np.float32)
    if dtype == "bf16":
        qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        return StepInputs(bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                          alpha, beta, dtype, qb, kb, vb)
    assert dtype == "f32"
    return StepInputs(q, k, v, alpha, beta, dtype)


def draw_gate(B: int, hv: int, d: int, *, seed: int, step: int, layer: int = 0,
              mu: float = 2.5, sigma: float = 1.5) -> np.ndarray:
    """Per-key-row gate [B][Hv][d] fp32 in logical row order."""
    g = rng_for(seed, _TAG_GATE, layer, step)
    x = g.normal(mu, sigma, size=(B, hv, d))
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def workload_inputs(w: Workload, step: int, *, calibration: bool = False, layer: int = 0,
                    B: int | None = None) -> StepInputs:
    seed = w.calib_seed if calibration else w.seed
    assert seed is not None
    return draw_inputs(B or w.B, w.hk, w.hv, w.d, dtype=w.dtype, seed=seed, step=step,
                       alpha_lo=w.alpha_lo, layer=layer)


def initial_state(w: Workload, *, layer: int = 0, B: int | None = None) -> np.ndarray:
    """S0 [B][Hv][d][d] fp32 following the workload's law."""
    B = B or w.B
    shape = (B, w.hv, w.d, w.d)
    if w.s0 == "zero":
        return np.zeros(shape, np.float32)
    g = rng_for(w.seed, _TAG_S0, layer)
    S = g.standard_normal(shape, dtype=np.float32)
    if w.s0 == "normal":
        S *= np.float32(w.s0_scale)
        return S
    assert w.s0 == "outlier"
    # per-head row and column factors, shared across sequences (Sec. 4.2 outliers)
    a = g.lognormal(0.0, w.outlier_sigma, size=(w.hv, w.d, 1)).astype(np.float32)
    e = g.lognormal(0.0, w.outlier_sigma, size=(w.hv, 1, w.d)).astype(np.float32)
    S *= a[None]
    S *= e[None]
    return S


def random_states(n: int, hv: int, d: int, *, seed: int, scale: float = 1.0,
                  outlier_sigma: float = 1.0) -> np.ndarray:
    """Arbitrary fp32 states [n][Hv][d][d] with row/column outliers (for pack
    and calibration parity)."""
    g = rng_for(seed, _TAG_RECORDS)
    S = g.standard_normal((n, hv, d, d), dtype=np.float32) * np.float32(scale)
    a = g.lognormal(0.0, outlier_sigma, size=(1, hv, d, 1)).astype(np.float32)
    e = g.lognormal(0.0, outlier_sigma, size=(1, hv, 1, d)).astype(np.float32)
    return (S * a * e).astype(np.float32)


@dataclass
class PackedState:
    pool8: np.ndarray  # int8  [B][Hv][n8][d]
    pool4: np.ndarray  # uint8 [B][Hv][d-n8][d/2]
    r: np.ndarray  # f32   [B][Hv][d]   physical row order
    c: np.ndarray  # f32   [Hv][d]
    perm: np.ndarray  # i32   [Hv][d]   logical row of each physical row
    n8: int


def random_packed_state(B: int, hv: int, d: int, n8: int, *, seed: int,
                        c_one: bool = False, identity_perm: bool = False,
                        full_rows: bool = False,
                        r_log10_range: tuple[float, float] = (-2.0, 0.5)) -> PackedState:
    """A valid packed state drawn directly: codes uniform on the symmetric range
    of each row width, log-uniform row factors, log-normal column factors.
    With full_rows, one random entry of every row is set to +-(top code) so
    that every row spans its whole range."""
    g = rng_for(seed, _TAG_PACKED)
    pool8 = g.integers(-127, 128, size=(B, hv, n8, d), dtype=np.int16).astype(np.int8)
    nib = g.integers(-7, 8, size=(B, hv, d - n8, d), dtype=np.int16).astype(np.int8)
    if full_rows:
        for arr, top in ((pool8, 127), (nib, 7)):
            if arr.size:
                col = g.integers(0, d, size=arr.shape[:-1])
                sign = np.where(g.random(arr.shape[:-1]) < 0.5, -1, 1).astype(np.int8)
                np.put_along_axis(arr, col[..., None], (sign * top)[..., None], axis=-1)
    lo = nib[..., 0::2].astype(np.uint8) & 0x0F
    hi = nib[..., 1::2].astype(np.uint8) & 0x0F
    pool4 = (lo | (hi << 4)).astype(np.uint8)
    r = (10.0 ** g.uniform(*r_log10_range, size=(B, hv, d))).astype(np.float32)
    if c_one:
        c = np.ones((hv, d), np.float32)
    else:
        c = g.lognormal(0.0, 1.0, size=(hv, d)).astype(np.float32)
    if identity_perm:
        perm = np.tile(np.arange(d, dtype=np.int32), (hv, 1))
    else:
        perm = np.stack([g.permutation(d).astype(np.int32) for _ in range(hv)])
    return PackedState(pool8, pool4, r, c, perm, n8)


def unpack_codes(ps_pool8: np.ndarray, ps_pool4: np.ndarray) -> np.ndarray:
    """Codes of every physical row as int8 [B][Hv][d][d] (layout read-out for
    test statistics; not part of any arithmetic)."""
    lo = (ps_pool4 & 0x0F).astype(np.int8)
    hi = (ps_pool4 >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)
    hi = np.where(hi >= 8, hi - 16, hi).astype(np.int8)
    z4 = np.empty(ps_pool4.shape[:-1] + (ps_pool4.shape[-1] * 2,), np.int8)
    z4[..., 0::2] = lo
    z4[..., 1::2] = hi
    return np.concatenate([ps_pool8, z4], axis=-2)


RAGGED_ROW_BYTES = (lambda d: 2 * d, lambda d: d, lambda d: 3 * d // 4, lambda d: d // 2,
                    lambda d: d // 4)


def ragged_segments(counts: np.ndarray, d: int) -> np.ndarray:
    """Byte offset of each head's segment in a slot of the ragged byte pool
    (segments padded to 16 bytes, heads in order)."""
    off, out = 0, []
    for h in range(counts.shape[0]):
        out.append(off)
        seg = sum(int(counts[h, k]) * RAGGED_ROW_BYTES[k](d) for k in range(5))
        off += (seg + 15) // 16 * 16
    return np.array(out, np.int64)


def unpack_ragged(pool: np.ndarray, counts: np.ndarray, d: int):
    """Read a ragged byte pool [B][slot_bytes] back into (codes, half_bits,
    cls): codes int32 [B][Hv][d][d] of the integer rows (physical order, 0
    on pivot rows), half_bits uint16 [B][Hv][d][d] of the pivot rows (0
    elsewhere) and the class of every physical row [Hv][d] (layout read-out
    for test statistics; not part of any arithmetic)."""
    B = pool.shape[0]
    hv = counts.shape[0]
    seg = ragged_segments(counts, d)
    codes = np.zeros((B, hv, d, d), np.int32)
    halfs = np.zeros((B, hv, d, d), np.uint16)
    cls = np.zeros((hv, d), np.int32)
    j = np.arange(d)
    for h in range(hv):
        off = int(seg[h])
        p = 0
        for k in range(5):
            rb = RAGGED_ROW_BYTES[k](d)
            for _ in range(int(counts[h, k])):
                row = pool[:, off:off + rb]
                cls[h, p] = k
                if k == 0:
                    halfs[:, h, p] = row.view(np.uint16) if row.flags["C_CONTIGUOUS"] else \
                        np.ascontiguousarray(row).view(np.uint16)
                elif k == 1:
                    codes[:, h, p] = row.view(np.int8)
                else:
                    if k == 2:
                        lo = (row[:, j // 2] >> (4 * (j % 2))) & 0xF
                        hi = (row[:, d // 2 + j // 4] >> (2 * (j % 4))) & 0x3
                        u = (lo | (hi << 4)).astype(np.int32)
                        codes[:, h, p] = np.where(u >= 32, u - 64, u)
                    elif k == 3:
                        u = ((row[:, j // 2] >> (4 * (j % 2))) & 0xF).astype(np.int32)
                        codes[:, h, p] = np.where(u >= 8, u - 16, u)
                    else:
                        u = ((row[:, j // 4] >> (2 * (j % 4))) & 0x3).astype(np.int32)
                        codes[:, h, p] = np.where(u >= 2, u - 4, u)
                off += rb
                p += 1
    return codes, halfs, cls


def random_ragged_counts(hv: int, d: int, *, seed: int, pivots: int = 1) -> np.ndarray:
    """Random class counts [Hv][5] (FP16, 8, 6, 4, 2 bits) summing to d, with
    `pivots` FP16 rows per head and every integer class present when d allows."""
    g = rng_for(seed, _TAG_PACKED, 5)
    counts = np.zeros((hv, 5), np.int32)
    for h in range(hv):
        rest = d - pivots
        cut = np.sort(g.integers(1, rest, size=3)) if rest > 4 else np.array([rest] * 3)
        counts[h] = [pivots, cut[0], cut[1] - cut[0], cut[2] - cut[1], rest - cut[2]]
    return counts


def calibration_shaped_counts(hv: int, d: int, *, seed: int, two_bit_heads: int = 0) -> np.ndarray:
    """Class counts [Hv][5] shaped like an assignment at a 6-bit budget: 0-3
    FP16 rows, about a fifth of the rows at 8 and at 4 bits, the rest 6-bit;
    the first `two_bit_heads` heads also get a few 2-bit rows.  Boundaries
    fall anywhere, so row groups straddle classes as they do after a real
    assignment."""
    g = rng_for(seed, _TAG_PACKED, 6)
    counts = np.zeros((hv, 5), np.int32)
    for h in range(hv):
        piv = int(g.integers(0, 4))
        n8 = int(g.integers(d // 8, d // 4 + 1))
        n4 = int(g.integers(d // 8, d // 4 + 1))
        n2 = int(g.integers(1, d // 8 + 1)) if h < two_bit_heads else 0
        counts[h] = [piv, n8, d - piv - n8 - n4 - n2, n4, n2]
    return counts


def random_ragged_state(B: int, counts: np.ndarray, d: int, slot_bytes: int, *, seed: int,
                        r_log10_range: tuple[float, float] = (-2.0, 0.5)):
    """A valid ragged packed state drawn directly (layout of the ragged
    formats: per head, FP16 rows, then 8-, 6-, 4-, 2-bit rows, segments
    padded to 16 bytes): integer codes uniform on each width's symmetric
    range, FP16 rows N(0, 1) rounded to binary16, log-uniform row factors
    (0 on FP16 rows).  Returns (pool uint8 [B][slot_bytes], r f32 [B][Hv][d])."""
    g = rng_for(seed, _TAG_PACKED, 7)
    hv = counts.shape[0]
    pool = np.zeros((B, slot_bytes), np.uint8)
    r = (10.0 ** g.uniform(*r_log10_range, size=(B, hv, d))).astype(np.float32)
    seg = ragged_segments(counts, d)
    assert seg[-1] + sum(int(counts[-1, k]) * RAGGED_ROW_BYTES[k](d) for k in range(5)) \
        <= slot_bytes
    qmax = (0, 127, 31, 7, 1)
    for h in range(hv):
        off = int(seg[h])
        p = 0
        for k in range(5):
            n = int(counts[h, k])
            if n == 0:
                continue
            rb = RAGGED_ROW_BYTES[k](d)
            if k == 0:
                vals = g.standard_normal((B, n, d)).astype(np.float16)
                rows = vals.view(np.uint8).reshape(B, n, 2 * d)
                r[:, h, p:p + n] = 0.0
            else:
                z = g.integers(-qmax[k], qmax[k] + 1, size=(B, n, d), dtype=np.int16)
                u = (z & ((1 << (8 if k == 1 else (6, 4, 2)[k - 2])) - 1)).astype(np.uint8)
                if k == 1:
                    rows = u
                elif k == 3:
                    rows = (u[..., 0::2] & 0xF) | ((u[..., 1::2] & 0xF) << 4)
                else:
                    f = (u >> 4) & 0x3 if k == 2 else u & 0x3  # the 2-bit fields
                    fields = (f[..., 0::4] | (f[..., 1::4] << 2) | (f[..., 2::4] << 4)
                              | (f[..., 3::4] << 6)).astype(np.uint8)
                    if k == 2:
                        nib = (u[..., 0::2] & 0xF) | ((u[..., 1::2] & 0xF) << 4)
                        rows = np.concatenate([nib, fields], axis=-1)
                    else:
                        rows = fields
            pool[:, off:off + n * rb] = rows.reshape(B, n * rb)
            off += n * rb
            p += n
    return pool, r
