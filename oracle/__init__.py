"""CPU oracle for the quantized gated delta-rule decode step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this package; the product library never does.

The arithmetic lives in ``stq_oracle.c`` (plain loops, IEEE double, built with
``-ffp-contract=off``); this module only builds it and marshals numpy arrays.
Every function below states the passage of the STEPQuant paper it follows
("STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State
Quantization", arXiv 2609.38169).

Parity status of each function (what pins it is in ``tests/test_oracle_pins.py``):
  rhe            pinned: numpy's rint on a half-integer grid (library routine)
  dequant        pinned: hand-made golden layout fixture, quantizer round trip
  pack           pinned: round trip, half-step error bound, S=0 closed form
  step           pinned: fixed point, delta-write closed form (o = v),
                 Proposition 1 identity, half-step bound, S0 = 0 closed form
  fp_step        pinned: App. B.1 norm identity, App. B.3 isolated-row read error
  calib_*        pinned: numpy max / stable argsort (library routines)
  pack_refit,    pinned: exact recovery of the column factors of an exactly
  step_refit,            representable state, covariance under column scaling,
  dequant_cs             weighted least-squares optimality (App. C.1 objective),
                         zero-column rule, fixed point
  impact_*       pinned: closed forms for unit-vector keys and queries
  alloc_*        (ragged row classes, FP16 pivots, lifetime-aware assignment;
                 ``stq_alloc_oracle.c``) pinned in ``tests/test_oracle_alloc_pins.py``:
                 equivalence with the 4/8-bit format, brute-force round trips
                 per class, numpy float16 rounding, step closed forms,
                 brute-force optimality of the assignment on small cases
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "stq_oracle.c"
_ALLOC_SRC = _HERE / "stq_alloc_oracle.c"
_LIB = _HERE / "libstq_oracle.so"


def compile_oracle(src: Path, out: Path, alloc_src: Path | None = None) -> Path:
    """Compile the oracle sources with gcc (plain C, no GPU code): ``src`` in
    place of ``stq_oracle.c`` and ``alloc_src`` (default: the real one) in
    place of ``stq_alloc_oracle.c``."""
    tmp = out.with_suffix(".so.tmp")
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
         "-Wall", "-o", str(tmp), str(src), str(alloc_src or _ALLOC_SRC), "-lm", "-lpthread"],
        check=True)
    os.replace(tmp, out)
    return out


def _stale() -> bool:
    if not _LIB.exists():
        return True
    t = _LIB.stat().st_mtime
    return t < _SRC.stat().st_mtime or t < _ALLOC_SRC.stat().st_mtime


def build(force: bool = True) -> Path:
    """Build ``libstq_oracle.so`` next to its sources."""
    if force or _stale():
        compile_oracle(_SRC, _LIB)
    return _LIB


def _bind(path: Path):
    lib = ctypes.CDLL(str(path))
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    lib.oracle_rhe.argtypes = [ctypes.c_double]
    lib.oracle_rhe.restype = ctypes.c_double
    lib.oracle_dequant.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I]
    lib.oracle_pack.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I]
    lib.oracle_step.argtypes = [I, I, I, I, I, I] + [P] * 15 + [I]
    lib.oracle_fp_step.argtypes = [I, I, I, I, I] + [P] * 7 + [I]
    lib.oracle_calib_cols.argtypes = [L, I, I, I, P, P]
    lib.oracle_calib_rows.argtypes = [L, I, I, I, P, P]
    lib.oracle_calib_finalize.argtypes = [I, I, I, I, P, P, P, P]
    lib.oracle_dequant_cs.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I]
    lib.oracle_pack_refit.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I]
    lib.oracle_step_refit.argtypes = [I, I, I, I, I, I] + [P] * 17 + [I]
    lib.oracle_impact_accumulate.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.oracle_impact_weights.argtypes = [I, I, P, P]
    lib.oracle_step_gated.argtypes = [I, I, I, I, I, I] + [P] * 15 + [I]
    lib.oracle_fp_step_gated.argtypes = [I, I, I, I, I] + [P] * 7 + [I]
    lib.oracle_step_refit_gated.argtypes = [I, I, I, I, I, I] + [P] * 17 + [I]
    lib.oracle_impact_accumulate_gated.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.oracle_f16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_f16_from_double.restype = ctypes.c_uint16
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_alloc_layout.argtypes = [I, I, P, P]
    lib.oracle_alloc_layout.restype = L
    lib.oracle_alloc_dequant.argtypes = [I, I, I, L, P, P, P, P, P, P, P, I]
    lib.oracle_alloc_pack.argtypes = [I, I, I, L, P, P, P, P, P, P, P, P, I]
    lib.oracle_alloc_step.argtypes = [I, I, I, I, L] + [P] * 18 + [I]
    lib.oracle_alloc_distortion.argtypes = [L, I, I, P, P, P]
    lib.oracle_alloc_lifetime.argtypes = [I, I, P, ctypes.c_double, I, P]
    lib.oracle_alloc_assign.argtypes = [I, I, P, P, I, I, I, P, P, P]
    for name in ("oracle_alloc_dequant", "oracle_alloc_pack", "oracle_alloc_step",
                 "oracle_alloc_distortion", "oracle_alloc_lifetime", "oracle_alloc_assign"):
        getattr(lib, name).restype = I
    for name in ("oracle_dequant", "oracle_pack", "oracle_step", "oracle_fp_step",
                 "oracle_calib_cols", "oracle_calib_rows", "oracle_calib_finalize",
                 "oracle_dequant_cs", "oracle_pack_refit", "oracle_step_refit",
                 "oracle_impact_accumulate", "oracle_impact_weights", "oracle_step_gated",
                 "oracle_fp_step_gated", "oracle_step_refit_gated",
                 "oracle_impact_accumulate_gated"):
        getattr(lib, name).restype = I
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class Oracle:
    """The oracle's entry points bound to one compiled library (the default one,
    or a deliberately broken copy in the mutation tests)."""

    def __init__(self, path: Path | None = None):
        self._path = path
        self._lib = None

    def lib(self):
        if self._lib is None:
            if self._path is None:
                if _stale():
                    build(force=True)
                self._path = _LIB
            self._lib = _bind(self._path)
        return self._lib

    def rhe(self, y: float) -> float:
        """Round half to even (Sec. 2.2 'round', reading R1)."""
        return self.lib().oracle_rhe(float(y))

    def dequant(self, pool8, pool4, r, c, perm, *, n8: int, nthreads: int = 1) -> np.ndarray:
        """Reconstruct S_ij = r_i c_j z_ij in logical row order (Sec. 4.3).

        pool8 [B][Hv][n8][dv] int8, pool4 [B][Hv][dk-n8][dv/2] uint8,
        r [B][Hv][dk] f32, c [Hv][dv] f32, perm [Hv][dk] i32 -> S [B][Hv][dk][dv] f64.
        """
        r = _c(r, np.float32)
        B, hv, dk = r.shape
        c = _c(c, np.float32)
        dv = c.shape[1]
        pool8 = _c(pool8, np.int8).reshape(B, hv, n8, dv)
        pool4 = _c(pool4, np.uint8).reshape(B, hv, dk - n8, dv // 2)
        perm = _c(perm, np.int32)
        S = np.empty((B, hv, dk, dv), np.float64)
        rc = self.lib().oracle_dequant(B, hv, dk, dv, n8, _ptr(pool8), _ptr(pool4), _ptr(r),
                                    _ptr(c), _ptr(perm), _ptr(S), nthreads)
        assert rc == 0
        return S

    def pack(self, S, c, perm, *, n8: int, nthreads: int = 1):
        """Requantize fp32 states S [B][Hv][dk][dv] (logical order) into the packed
        layout (Table C2 steps 4 and 6 applied to a given state).

        Returns (pool8, pool4, r)."""
        S = _c(S, np.float32)
        B, hv, dk, dv = S.shape
        c = _c(c, np.float32)
        perm = _c(perm, np.int32)
        pool8 = np.zeros((B, hv, n8, dv), np.int8)
        pool4 = np.zeros((B, hv, dk - n8, dv // 2), np.uint8)
        r = np.empty((B, hv, dk), np.float32)
        rc = self.lib().oracle_pack(B, hv, dk, dv, n8, _ptr(S), _ptr(c), _ptr(perm), _ptr(pool8),
                                 _ptr(pool4), _ptr(r), nthreads)
        assert rc == 0
        return pool8, pool4, r

    def step(self, pool8, pool4, r, c, perm, q, k, v, alpha, beta, *, n8: int,
             want_X: bool = False, nthreads: int = 1, gate=None):
        """One quantized decode step (Table C2; Sec. 2.1 Eq. (1) with D = alpha I).

        q, k [B][Hk][dk], v [B][Hv][dv], alpha, beta [B][Hv] (fp32 values; bf16
        inputs are passed widened).  Returns dict with pool8, pool4, r, o and,
        if want_X, the pre-requantization state X [B][Hv][dk][dv] (f64).  With
        gate [B][Hv][dk] (logical rows) the diagonal gate D = diag(gate) of the
        KDA form replaces alpha."""
        r = _c(r, np.float32)
        B, hv, dk = r.shape
        c = _c(c, np.float32)
        dv = c.shape[1]
        q = _c(q, np.float32)
        hk = q.shape[1]
        k = _c(k, np.float32)
        v = _c(v, np.float32)
        beta = _c(beta, np.float32)
        if gate is not None:
            g_or_a = _c(gate, np.float32)
            assert g_or_a.shape == (B, hv, dk)
        else:
            g_or_a = _c(alpha, np.float32)
            assert g_or_a.shape == (B, hv)
        assert q.shape == (B, hk, dk) and k.shape == (B, hk, dk)
        assert v.shape == (B, hv, dv) and beta.shape == (B, hv)
        pool8 = _c(pool8, np.int8).reshape(B, hv, n8, dv)
        pool4 = _c(pool4, np.uint8).reshape(B, hv, dk - n8, dv // 2)
        perm = _c(perm, np.int32)
        out = {
            "pool8": np.zeros_like(pool8),
            "pool4": np.zeros_like(pool4),
            "r": np.empty_like(r),
            "o": np.empty((B, hv, dv), np.float32),
        }
        X = np.empty((B, hv, dk, dv), np.float64) if want_X else None
        fn = self.lib().oracle_step_gated if gate is not None else self.lib().oracle_step
        rc = fn(B, hv, hk, dk, dv, n8, _ptr(pool8), _ptr(pool4), _ptr(r),
                                 _ptr(c), _ptr(perm), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(g_or_a), _ptr(beta), _ptr(out["pool8"]),
                                 _ptr(out["pool4"]), _ptr(out["r"]), _ptr(out["o"]),
                                 _ptr(X), nthreads)
        assert rc == 0
        if want_X:
            out["X"] = X
        return out

    def fp_step(self, S, q, k, v, alpha, beta, *, nthreads: int = 1, gate=None):
        """Unquantized gated delta-rule step (Sec. 2.1 Eq. (1), D = alpha I).

        S [B][Hv][dk][dv] f64 is updated IN PLACE; returns o [B][Hv][dv] f64."""
        assert S.dtype == np.float64 and S.flags["C_CONTIGUOUS"]
        B, hv, dk, dv = S.shape
        q = _c(q, np.float32)
        hk = q.shape[1]
        k = _c(k, np.float32)
        v = _c(v, np.float32)
        g_or_a = _c(gate if gate is not None else alpha, np.float32)
        beta = _c(beta, np.float32)
        o = np.empty((B, hv, dv), np.float64)
        fn = self.lib().oracle_fp_step_gated if gate is not None else self.lib().oracle_fp_step
        rc = fn(B, hv, hk, dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                _ptr(g_or_a), _ptr(beta), _ptr(o), nthreads)
        assert rc == 0
        return o

    def calib_cols(self, S, colmax):
        """colmax[h][j] <- max(colmax, max over records, rows of |S|).
        S [n_rec][Hv][dk][dv]; colmax [Hv][dv] f64, updated in place."""
        S = _c(S, np.float64)
        n, hv, dk, dv = S.shape
        assert colmax.dtype == np.float64 and colmax.shape == (hv, dv)
        assert self.lib().oracle_calib_cols(n, hv, dk, dv, _ptr(S), _ptr(colmax)) == 0

    def calib_rows(self, S, rowscore):
        """rowscore[h][i] += sum over records and columns of S^2."""
        S = _c(S, np.float64)
        n, hv, dk, dv = S.shape
        assert rowscore.dtype == np.float64 and rowscore.shape == (hv, dk)
        assert self.lib().oracle_calib_rows(n, hv, dk, dv, _ptr(S), _ptr(rowscore)) == 0

    def calib_finalize(self, colmax, rowscore, n8: int):
        """Return (c [Hv][dv] f32, perm [Hv][dk] i32) from the accumulated
        statistics: c = column absmax (0 -> 1); the n8 top-score rows (ties to the
        lower index) first in ascending order, then the rest ascending."""
        colmax = _c(colmax, np.float64)
        rowscore = _c(rowscore, np.float64)
        hv, dv = colmax.shape
        dk = rowscore.shape[1]
        c = np.empty((hv, dv), np.float32)
        perm = np.empty((hv, dk), np.int32)
        assert self.lib().oracle_calib_finalize(hv, dk, dv, n8, _ptr(colmax), _ptr(rowscore),
                                             _ptr(c), _ptr(perm)) == 0
        return c, perm


    # ---- per-state column factors with the online refit (App. C.1; Table C2
    # step 5; reading R14)
    def dequant_cs(self, pool8, pool4, r, cs, perm, *, n8: int, nthreads: int = 1):
        """S_ij = r_i cs_j z_ij with per-state column factors cs [B][Hv][dv]."""
        r = _c(r, np.float32)
        B, hv, dk = r.shape
        cs = _c(cs, np.float32)
        dv = cs.shape[2]
        pool8 = _c(pool8, np.int8).reshape(B, hv, n8, dv)
        pool4 = _c(pool4, np.uint8).reshape(B, hv, dk - n8, dv // 2)
        perm = _c(perm, np.int32)
        S = np.empty((B, hv, dk, dv), np.float64)
        rc = self.lib().oracle_dequant_cs(B, hv, dk, dv, n8, _ptr(pool8), _ptr(pool4), _ptr(r),
                                          _ptr(cs), _ptr(perm), _ptr(S), nthreads)
        assert rc == 0
        return S

    def pack_refit(self, S, c0, perm, w2, *, n8: int, nthreads: int = 1):
        """Codes and row factors against c0 [Hv][dv], then the per-state column
        refit (weights w2 [Hv][dk], logical rows).  Returns pool8, pool4, r, cs."""
        S = _c(S, np.float32)
        B, hv, dk, dv = S.shape
        c0 = _c(c0, np.float32)
        perm = _c(perm, np.int32)
        w2 = _c(w2, np.float32)
        pool8 = np.zeros((B, hv, n8, dv), np.int8)
        pool4 = np.zeros((B, hv, dk - n8, dv // 2), np.uint8)
        r = np.empty((B, hv, dk), np.float32)
        cs = np.empty((B, hv, dv), np.float32)
        rc = self.lib().oracle_pack_refit(B, hv, dk, dv, n8, _ptr(S), _ptr(c0), _ptr(perm),
                                          _ptr(w2), _ptr(pool8), _ptr(pool4), _ptr(r), _ptr(cs),
                                          nthreads)
        assert rc == 0
        return pool8, pool4, r, cs

    def step_refit(self, pool8, pool4, r, cs, perm, w2, q, k, v, alpha, beta, *, n8: int,
                   want_X: bool = False, nthreads: int = 1, gate=None):
        """One decode step with per-state column factors and the online column
        refit (Table C2 steps 1-6).  Returns dict pool8, pool4, r, cs, o (and X)."""
        r = _c(r, np.float32)
        B, hv, dk = r.shape
        cs = _c(cs, np.float32)
        dv = cs.shape[2]
        q = _c(q, np.float32)
        hk = q.shape[1]
        k = _c(k, np.float32)
        v = _c(v, np.float32)
        g_or_a = _c(gate if gate is not None else alpha, np.float32)
        beta = _c(beta, np.float32)
        pool8 = _c(pool8, np.int8).reshape(B, hv, n8, dv)
        pool4 = _c(pool4, np.uint8).reshape(B, hv, dk - n8, dv // 2)
        perm = _c(perm, np.int32)
        w2 = _c(w2, np.float32)
        out = {"pool8": np.zeros_like(pool8), "pool4": np.zeros_like(pool4),
               "r": np.empty_like(r), "cs": np.empty_like(cs),
               "o": np.empty((B, hv, dv), np.float32)}
        X = np.empty((B, hv, dk, dv), np.float64) if want_X else None
        fn = self.lib().oracle_step_refit_gated if gate is not None else self.lib().oracle_step_refit
        rc = fn(
            B, hv, hk, dk, dv, n8, _ptr(pool8), _ptr(pool4), _ptr(r), _ptr(cs), _ptr(perm),
            _ptr(w2), _ptr(q), _ptr(k), _ptr(v), _ptr(g_or_a), _ptr(beta), _ptr(out["pool8"]),
            _ptr(out["pool4"]), _ptr(out["r"]), _ptr(out["cs"]), _ptr(out["o"]), _ptr(X),
            nthreads)
        assert rc == 0
        if want_X:
            out["X"] = X
        return out

    def impact_accumulate(self, q, k, alpha, beta, omega, *, hv: int, gate=None):
        """omega[h][i] += sum over the batch of (alpha (q_i - beta k_i k.q))^2
        (Sec. 4.1 row impact with the scalar gate; App. C.1).  omega [Hv][dk] f64."""
        q = _c(q, np.float32)
        B, hk, dk = q.shape
        k = _c(k, np.float32)
        g_or_a = _c(gate if gate is not None else alpha, np.float32)
        beta = _c(beta, np.float32)
        assert omega.dtype == np.float64 and omega.shape == (hv, dk)
        fn = (self.lib().oracle_impact_accumulate_gated if gate is not None
              else self.lib().oracle_impact_accumulate)
        assert fn(B, hv, hk, dk, _ptr(q), _ptr(k), _ptr(g_or_a), _ptr(beta), _ptr(omega)) == 0

    def impact_weights(self, omega):
        """Squared row-impact weights w2 = (omega / mean omega)^(1/4) per head
        (App. B.3: w proportional to omega^(1/8)), floored at 2^-32; an
        all-zero head gives 1."""
        omega = _c(omega, np.float64)
        hv, dk = omega.shape
        w2 = np.empty((hv, dk), np.float32)
        assert self.lib().oracle_impact_weights(hv, dk, _ptr(omega), _ptr(w2)) == 0
        return w2


    # ------------------------------------------------ ragged row classes --
    # stq_alloc_oracle.c; classes k = 0..4 are FP16 pivots, 8, 6, 4, 2 bits.

    def f16(self, x: float) -> int:
        """IEEE binary16 bits of x, nearest even, saturating (reading R18)."""
        return int(self.lib().oracle_f16_from_double(float(x)))

    def f16_value(self, h: int) -> float:
        return float(self.lib().oracle_f16_to_double(int(h)))

    def alloc_layout(self, counts, d: int):
        """Per-head segment offsets [Hv] and the bytes one slot needs
        (App. C.3 Table C2 storage; reading R17)."""
        counts = _c(counts, np.int32)
        hv = counts.shape[0]
        off = np.zeros(hv, np.int64)
        need = self.lib().oracle_alloc_layout(hv, d, _ptr(counts), _ptr(off))
        assert need >= 0, "row-class counts must sum to d"
        return off, int(need)

    def alloc_dequant(self, pool, r, counts, perm, *, c=None, cs=None, nthreads: int = 1):
        """S [B][Hv][d][d] (logical order) from the ragged pool [B][slot_bytes]
        (Table C2 step 1; readings R17-R19)."""
        pool = _c(pool, np.uint8)
        r = _c(r, np.float32)
        B, hv, d = r.shape
        counts = _c(counts, np.int32)
        perm = _c(perm, np.int32)
        S = np.empty((B, hv, d, d), np.float64)
        c = None if c is None else _c(c, np.float32)
        cs = None if cs is None else _c(cs, np.float32)
        rc = self.lib().oracle_alloc_dequant(
            B, hv, d, pool.shape[1], _ptr(counts), _ptr(perm), _ptr(pool), _ptr(r),
            _ptr(c), _ptr(cs), _ptr(S), nthreads)
        assert rc == 0
        return S

    def alloc_pack(self, S, counts, perm, c, slot_bytes: int, *, w2=None, refit=False,
                   nthreads: int = 1):
        """Pack S [B][Hv][d][d] into a ragged pool [B][slot_bytes]; returns
        (pool, r) or, with refit, (pool, r, cs) (readings R17-R19, R14)."""
        S = _c(S, np.float64)
        B, hv, d, _ = S.shape
        counts = _c(counts, np.int32)
        perm = _c(perm, np.int32)
        c = _c(c, np.float32)
        pool = np.zeros((B, slot_bytes), np.uint8)
        r = np.zeros((B, hv, d), np.float32)
        cs = np.zeros((B, hv, d), np.float32) if refit else None
        w2 = None if w2 is None else _c(w2, np.float32)
        rc = self.lib().oracle_alloc_pack(
            B, hv, d, slot_bytes, _ptr(counts), _ptr(perm), _ptr(S), _ptr(c), _ptr(w2),
            _ptr(pool), _ptr(r), _ptr(cs), nthreads)
        assert rc == 0
        return (pool, r, cs) if refit else (pool, r)

    def alloc_step(self, pool, r, counts, perm, q, k, v, alpha, beta, *, c=None, cs=None,
                   w2=None, gate=None, want_X: bool = False, nthreads: int = 1):
        """One decode step on the ragged format (Table C2 with pivots; Eq. (1)
        with the scalar or, given gate [B][Hv][d], the row gate).  Fixed c
        [Hv][d], or per-state cs [B][Hv][d] with the refit (w2 needed).
        Returns dict pool, r, o (and cs, X)."""
        pool = _c(pool, np.uint8)
        r = _c(r, np.float32)
        B, hv, d = r.shape
        q = _c(q, np.float32)
        hk = q.shape[1]
        counts = _c(counts, np.int32)
        perm = _c(perm, np.int32)
        out = {"pool": np.zeros_like(pool), "r": np.zeros_like(r),
               "o": np.empty((B, hv, d), np.float32)}
        if cs is not None:
            out["cs"] = np.zeros((B, hv, d), np.float32)
        X = np.empty((B, hv, d, d), np.float64) if want_X else None
        opt = lambda a: None if a is None else _c(a, np.float32)  # noqa: E731
        # every converted array is held by a name until the call returns
        c, cs, w2, alpha, gate = opt(c), opt(cs), opt(w2), opt(alpha), opt(gate)
        k, v, beta = _c(k, np.float32), _c(v, np.float32), _c(beta, np.float32)
        rc = self.lib().oracle_alloc_step(
            B, hv, hk, d, pool.shape[1], _ptr(counts), _ptr(perm), _ptr(pool), _ptr(r),
            _ptr(c), _ptr(cs), _ptr(w2), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(gate),
            _ptr(beta), _ptr(out["pool"]), _ptr(out["r"]), _ptr(out.get("cs")), _ptr(out["o"]),
            _ptr(X), nthreads)
        assert rc == 0
        if want_X:
            out["X"] = X
        return out

    def alloc_distortion(self, S, c, dist):
        """dist [Hv][d][5] += candidate distortions of the records S
        [n][Hv][d][d] (App. A.3 KDA distortion; reading R20)."""
        S = _c(S, np.float64)
        n, hv, d, _ = S.shape
        assert dist.dtype == np.float64 and dist.shape == (hv, d, 5)
        c = _c(c, np.float32)
        assert self.lib().oracle_alloc_distortion(n, hv, d, _ptr(S), _ptr(c), _ptr(dist)) == 0

    def alloc_lifetime(self, logret, n: float, horizon: int):
        """L [Hv][d] from the summed log retention over n samples (App. A.3;
        reading R21)."""
        logret = _c(logret, np.float64)
        Lw = np.empty_like(logret)
        assert self.lib().oracle_alloc_lifetime(logret.shape[0], logret.shape[1], _ptr(logret),
                                                float(n), int(horizon), _ptr(Lw)) == 0
        return Lw

    def alloc_assign(self, dist, Lw, *, nominal: int, n_pivot: int, candidates=(8, 6, 4)):
        """Pivots and widths per row (App. C.2; readings R22, R23).  Returns
        bits [Hv][d], counts [Hv][5], perm [Hv][d]."""
        dist = _c(dist, np.float64)
        hv, d, _ = dist.shape
        Lw = _c(Lw, np.float64)
        mask = 0
        for b in candidates:
            mask |= 1 << {8: 1, 6: 2, 4: 3, 2: 4}[b]
        bits = np.zeros((hv, d), np.int32)
        counts = np.zeros((hv, 5), np.int32)
        perm = np.zeros((hv, d), np.int32)
        rc = self.lib().oracle_alloc_assign(hv, d, _ptr(dist), _ptr(Lw), mask, nominal, n_pivot,
                                            _ptr(bits), _ptr(counts), _ptr(perm))
        assert rc == 0, "infeasible budget or bad candidates"
        return bits, counts, perm


_default = Oracle()
rhe = _default.rhe
dequant = _default.dequant
pack = _default.pack
step = _default.step
fp_step = _default.fp_step
calib_cols = _default.calib_cols
calib_rows = _default.calib_rows
calib_finalize = _default.calib_finalize
dequant_cs = _default.dequant_cs
pack_refit = _default.pack_refit
step_refit = _default.step_refit
impact_accumulate = _default.impact_accumulate
impact_weights = _default.impact_weights
f16 = _default.f16
f16_value = _default.f16_value
alloc_layout = _default.alloc_layout
alloc_dequant = _default.alloc_dequant
alloc_pack = _default.alloc_pack
alloc_step = _default.alloc_step
alloc_distortion = _default.alloc_distortion
alloc_lifetime = _default.alloc_lifetime
alloc_assign = _default.alloc_assign
