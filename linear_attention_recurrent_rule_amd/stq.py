"""Thin ctypes binding of libstq.so (include/stq.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libstq.so.  PyTorch provides device memory and the current stream.
There is no fallback: if libstq.so is missing the import of the library fails
loudly, and every call on tensors that are not on a HIP device is rejected.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

import numpy as np
import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libstq.so"

STQ_OK = 0
STATUS_NAMES = {0: "STQ_OK", 1: "STQ_E_ARG", 2: "STQ_E_SHAPE", 3: "STQ_E_UNSUPPORTED",
                4: "STQ_E_SPACE", 5: "STQ_E_STATE", 6: "STQ_E_DEVICE"}

FMT_MIXED48, FMT_INT8ROW, FMT_FP32, FMT_REFIT, FMT_ALLOC, FMT_ALLOC_REFIT = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
OUT_BF16 = 0x100  # readout written in bf16 (STQ_OUT_BF16)
CAL_RESET, CAL_COLS, CAL_ROWS, CAL_FINALIZE, CAL_DIST = 1, 2, 4, 8, 16
# ragged row classes (ALLOC formats): FP16 pivots, 8, 6, 4, 2 bits
CLASS_BITS = (16, 8, 6, 4, 2)
LAYOUT_STRIDE = 8
CAL_CHUNKS = 64


class StqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib().stq_status_str(status).decode()}")


class Desc(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("n_heads_v", ctypes.c_int32),
                ("n_heads_k", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("n8", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("nominal_bits", ctypes.c_int32), ("n_pivot", ctypes.c_int32)]


class CState(ctypes.Structure):
    _fields_ = [("desc", Desc), ("pool8", ctypes.c_void_p), ("pool4", ctypes.c_void_p),
                ("r", ctypes.c_void_p), ("c", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("colmax", ctypes.c_void_p), ("rowscore", ctypes.c_void_p),
                ("cal_colpart", ctypes.c_void_p), ("cal_rowpart", ctypes.c_void_p),
                ("s32", ctypes.c_void_p), ("cs", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("impact", ctypes.c_void_p), ("layout", ctypes.c_void_p),
                ("dist", ctypes.c_void_p), ("logret", ctypes.c_void_p), ("nret", ctypes.c_void_p),
                ("slot_bytes", ctypes.c_int64), ("calibrated", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_LIB = None
EXPORTS = ("stq_state_bytes", "stq_alloc_state", "stq_calibrate", "stq_calibrate_impact",
           "stq_calibrate_impact_gated", "stq_set_calibration", "stq_pack_state",
           "stq_decode_step", "stq_decode_step_into", "stq_decode_step_gated",
           "stq_dequant_state", "stq_stream_copy", "stq_status_str", "stq_abi_version",
           "stq_calibrate_retention", "stq_allocate", "stq_set_alloc_layout",
           "stq_assign_rows", "stq_calibrate_static")


def _lib():
    global _LIB
    if _LIB is None:
        if not LIB_PATH.exists():
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_recurrent_rule_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(str(LIB_PATH))
        P, I32, I64, U32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_uint32, ctypes.c_size_t)
        lib.stq_state_bytes.argtypes = [ctypes.POINTER(Desc)]
        lib.stq_state_bytes.restype = SZ
        lib.stq_alloc_state.argtypes = [ctypes.POINTER(Desc), P, SZ, P, ctypes.POINTER(CState)]
        lib.stq_calibrate.argtypes = [ctypes.POINTER(CState), P, I64, U32, P]
        lib.stq_calibrate_static.argtypes = lib.stq_calibrate.argtypes
        lib.stq_set_calibration.argtypes = [ctypes.POINTER(CState), P, P, P]
        lib.stq_calibrate_impact.argtypes = [ctypes.POINTER(CState), P, P, I32, P, P, I32, U32, P]
        lib.stq_calibrate_impact_gated.argtypes = lib.stq_calibrate_impact.argtypes
        lib.stq_pack_state.argtypes = [ctypes.POINTER(CState), P, P, I32, P]
        lib.stq_decode_step.argtypes = [ctypes.POINTER(CState), P, I32, P, P, P, I32, P, P, P, P]
        lib.stq_decode_step_into.argtypes = [ctypes.POINTER(CState), ctypes.POINTER(CState), P,
                                             I32, P, P, P, I32, P, P, P, P]
        lib.stq_decode_step_gated.argtypes = lib.stq_decode_step_into.argtypes
        lib.stq_calibrate_retention.argtypes = [ctypes.POINTER(CState), P, P, I32, U32, P]
        lib.stq_allocate.argtypes = [ctypes.POINTER(CState), I32, U32, P]
        lib.stq_set_alloc_layout.argtypes = [ctypes.POINTER(CState), P, P, P, P]
        lib.stq_assign_rows.argtypes = [I32, I32, P, P, ctypes.c_double, I32, U32, I32, I32, P,
                                        P]
        lib.stq_dequant_state.argtypes = [ctypes.POINTER(CState), P, I32, P, P]
        lib.stq_stream_copy.argtypes = [P, P, SZ, P]
        lib.stq_status_str.argtypes = [I32]
        lib.stq_status_str.restype = ctypes.c_char_p
        lib.stq_abi_version.restype = I32
        for name in ("stq_alloc_state", "stq_calibrate", "stq_calibrate_impact",
                     "stq_calibrate_impact_gated", "stq_set_calibration",
                     "stq_pack_state", "stq_decode_step", "stq_decode_step_into",
                     "stq_decode_step_gated", "stq_dequant_state", "stq_stream_copy",
                     "stq_calibrate_retention", "stq_allocate", "stq_set_alloc_layout",
           "stq_assign_rows", "stq_calibrate_static"):
            getattr(lib, name).restype = I32
        _LIB = lib
    return _LIB


def lib():
    """The loaded libstq.so (raises ImportError if it has not been built)."""
    return _lib()


def _check(status: int, where: str):
    if status != STQ_OK:
        raise StqError(status, where)


# the current stream's handle straight from torch's C layer where it offers
# that (a Python Stream object costs microseconds per call)
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream=None, device=None):
    """Handle of `stream`, else of the current stream (on `device` when given,
    the device of the state being worked on)."""
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is not None and device is not None and device.index is not None:
        return _RAW_STREAM(device.index)
    return torch.cuda.current_stream().cuda_stream


_FLOAT_IN = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _check_meta(t, name: str, shape=None, dtypes=None):
    """Type, dtype (one of `dtypes`) and exact shape (an entry None matches any
    extent) of an argument; None passes."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtypes is not None and t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be {names}, got {str(t.dtype).replace('torch.', '')}")
    if shape is not None:
        ts = t.shape
        if None in shape:
            ok = len(ts) == len(shape) and all(e is None or n == e for n, e in zip(ts, shape))
        else:
            ok = ts == shape
        if not ok:
            want = "[" + "][".join("*" if e is None else str(e) for e in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")


def _dev_ptr(t: torch.Tensor | None, name: str, shape=None, dtypes=None, device=None):
    """Device pointer of `t` after checking it, so that a mismatch raises
    ValueError before anything is queued: dtype and shape as _check_meta, on a
    HIP device (on `device` when given), contiguous.  None passes through as
    NULL."""
    if t is None:
        return None
    _check_meta(t, name, shape, dtypes)
    return _placed_ptr(t, name, device)


def _placed_ptr(t: torch.Tensor | None, name: str, device=None):
    """The device checks of _dev_ptr (on a HIP device, on `device` when given,
    contiguous) and the pointer, as an integer for a c_void_p argument."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and (t.get_device() != device.index if device.index is not None
                               else t.device != device):
        raise ValueError(f"{name} is on {t.device}, the state on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dev_ptrs(*specs, device=None):
    """_dev_ptr over several (tensor, name, shape, dtypes) specs, with every
    dtype and shape checked before any device check, so that the first error
    names the argument that is wrong rather than the first one on the host."""
    for t, name, shape, dtypes in specs:
        _check_meta(t, name, shape, dtypes)
    return [_placed_ptr(t, name, device) for t, name, shape, dtypes in specs]


def _in_dtype(q, k, v) -> int:
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
    if q.dtype == torch.float32:
        dt = F32
    elif q.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise ValueError("q, k, v must be float32 or bfloat16")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    return dt


def _batch(t, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.dim() < 1:
        raise ValueError(f"{name} must be a tensor with a leading batch dimension")
    return int(t.shape[0])


def assign_rows(dist, logret, nret: float, horizon: int, nominal_bits: int, n_pivot: int,
                candidates: int = 0):
    """Pivots and row widths from statistics in host memory (stq_assign_rows):
    dist [Hv][d][5] and logret [Hv][d] (float64 arrays), nret the number of
    retention samples.  Returns counts [Hv][5] and perm [Hv][d] (int32)."""
    dist = np.asarray(dist)
    logret = np.asarray(logret)
    if dist.dtype != np.float64 or logret.dtype != np.float64:
        raise ValueError("dist and logret must be float64")
    if dist.ndim != 3 or dist.shape[2] != 5 or logret.shape != dist.shape[:2]:
        raise ValueError("dist must be [Hv][d][5] and logret [Hv][d]")
    dist = np.ascontiguousarray(dist)
    logret = np.ascontiguousarray(logret)
    hv, d = logret.shape
    counts = np.zeros((hv, 5), np.int32)
    perm = np.zeros((hv, d), np.int32)
    _check(_lib().stq_assign_rows(hv, d, dist.ctypes.data, logret.ctypes.data, float(nret),
                                  int(horizon), int(candidates), int(nominal_bits), int(n_pivot),
                                  counts.ctypes.data, perm.ctypes.data), "stq_assign_rows")
    return counts, perm


def state_bytes(n_slots, n_heads_v, n_heads_k, d, n8, fmt, nominal_bits=0, n_pivot=0) -> int:
    d_ = Desc(n_slots, n_heads_v, n_heads_k, d, d, n8, fmt, nominal_bits, n_pivot)
    return int(_lib().stq_state_bytes(ctypes.byref(d_)))


@dataclass
class Geometry:
    n_slots: int
    n_heads_v: int
    n_heads_k: int
    d: int
    n8: int
    fmt: int = FMT_MIXED48
    nominal_bits: int = 0  # ALLOC formats: integer budget per value
    n_pivot: int = 0       # ALLOC formats: FP16 pivot rows per slot


class State:
    """A packed recurrent-state pool carved from one torch-owned device buffer."""

    def __init__(self, geo: Geometry, device="cuda", stream=None):
        self.geo = geo
        self.desc = Desc(geo.n_slots, geo.n_heads_v, geo.n_heads_k, geo.d, geo.d, geo.n8, geo.fmt,
                         geo.nominal_bits, geo.n_pivot)
        nbytes = int(_lib().stq_state_bytes(ctypes.byref(self.desc)))
        if nbytes == 0:
            raise StqError(2, "stq_state_bytes (invalid or unsupported geometry)")
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._device = self.buffer.device  # (read once: a device object per call costs time)
        self.c_state = CState()
        _check(_lib().stq_alloc_state(ctypes.byref(self.desc), _dev_ptr(self.buffer, "buffer"),
                                      nbytes, _stream(stream, self._device), ctypes.byref(self.c_state)),
               "stq_alloc_state")

    # -- views into the caller-owned buffer (for inspection and tests) --
    def _view(self, field: str, dtype, shape):
        ptr = getattr(self.c_state, field)
        if not ptr:
            return None
        off = ptr - self.buffer.data_ptr()
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + nbytes].view(dtype).view(*shape)

    @property
    def pool8(self):
        g = self.geo
        return self._view("pool8", torch.int8, (g.n_slots, g.n_heads_v, g.n8, g.d))

    @property
    def pool4(self):
        g = self.geo
        return self._view("pool4", torch.uint8, (g.n_slots, g.n_heads_v, g.d - g.n8, g.d // 2))

    @property
    def r(self):
        g = self.geo
        return self._view("r", torch.float32, (g.n_slots, g.n_heads_v, g.d))

    @property
    def c(self):
        g = self.geo
        return self._view("c", torch.float32, (g.n_heads_v, g.d))

    @property
    def perm(self):
        g = self.geo
        return self._view("perm", torch.int32, (g.n_heads_v, g.d))

    @property
    def s32(self):
        g = self.geo
        return self._view("s32", torch.float32, (g.n_slots, g.n_heads_v, g.d, g.d))

    @property
    def colmax(self):
        g = self.geo
        return self._view("colmax", torch.float32, (g.n_heads_v, g.d))

    @property
    def rowscore(self):
        g = self.geo
        return self._view("rowscore", torch.float64, (g.n_heads_v, g.d))

    @property
    def cs(self):
        g = self.geo
        return self._view("cs", torch.float32, (g.n_slots, g.n_heads_v, g.d))

    @property
    def w2(self):
        g = self.geo
        return self._view("w2", torch.float32, (g.n_heads_v, g.d))

    @property
    def impact(self):
        g = self.geo
        return self._view("impact", torch.float64, (g.n_heads_v, g.d))

    # -- ragged row classes (ALLOC formats) --
    @property
    def pool(self):
        """The byte pool [n_slots][slot_bytes] of an ALLOC state."""
        g = self.geo
        return self._view("pool8", torch.uint8, (g.n_slots, int(self.c_state.slot_bytes)))

    @property
    def layout(self):
        g = self.geo
        return self._view("layout", torch.int32, (g.n_heads_v, LAYOUT_STRIDE))

    @property
    def dist(self):
        g = self.geo
        return self._view("dist", torch.float64, (g.n_heads_v, g.d, 5))

    @property
    def logret(self):
        g = self.geo
        return self._view("logret", torch.float64, (g.n_heads_v, g.d))

    @property
    def nret(self):
        g = self.geo
        return self._view("nret", torch.float64, (g.n_heads_v,))

    @property
    def slot_bytes(self) -> int:
        return int(self.c_state.slot_bytes)

    def calibrate_retention(self, alpha=None, gate=None, flags: int = 0, stream=None):
        """Fold one step's gates (alpha [B][Hv] or gate [B][Hv][d]) into the
        summed log retention (stq_calibrate_retention)."""
        g, dv = self.geo, self._device
        src = gate if gate is not None else alpha
        B = 0 if src is None else _batch(src, "gate" if gate is not None else "alpha")
        pa, pg = _dev_ptrs((alpha, "alpha", (B, g.n_heads_v), _F32),
                           (gate, "gate", (B, g.n_heads_v, g.d), _F32), device=dv)
        _check(_lib().stq_calibrate_retention(ctypes.byref(self.c_state), pa, pg, B, flags,
                                              _stream(stream, self._device)), "stq_calibrate_retention")

    def allocate(self, horizon: int, candidates: int = 0, stream=None):
        """Pivots and row widths from the calibration statistics (stq_allocate)."""
        _check(_lib().stq_allocate(ctypes.byref(self.c_state), int(horizon), int(candidates),
                                   _stream(stream, self._device)), "stq_allocate")

    def set_alloc_layout(self, counts, c: torch.Tensor, perm: torch.Tensor, stream=None):
        """Install class counts [Hv][5] (host array), c and perm (device)."""
        g, dv = self.geo, self._device
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        if cnt.shape != (g.n_heads_v, 5):
            raise ValueError(f"counts must have shape [{g.n_heads_v}][5], got {list(cnt.shape)}")
        if c is None or perm is None:
            raise ValueError("c and perm are required")
        pc, pp = _dev_ptrs((c, "c", (g.n_heads_v, g.d), _F32),
                           (perm, "perm", (g.n_heads_v, g.d), _I32), device=dv)
        _check(_lib().stq_set_alloc_layout(ctypes.byref(self.c_state), cnt.ctypes.data, pc, pp,
                                           _stream(stream, self._device)), "stq_set_alloc_layout")

    @property
    def calibrated(self) -> bool:
        return bool(self.c_state.calibrated)

    # -- entry points --
    def calibrate(self, records: torch.Tensor | None, flags: int, stream=None):
        """Fold fp32 records [n][Hv][d][d] (logical rows) into the statistics
        that `flags` name (stq_calibrate)."""
        g = self.geo
        n = 0 if records is None else _batch(records, "records")
        p = _dev_ptr(records, "records", (n, g.n_heads_v, g.d, g.d), _F32, self._device)
        _check(_lib().stq_calibrate(ctypes.byref(self.c_state), p, n, flags,
                                    _stream(stream, self._device)), "stq_calibrate")

    def calibrate_static(self, records: torch.Tensor | None, flags: int, stream=None):
        """stq_calibrate_static: as calibrate, with the partial results in the
        library's fixed per-GPU array (allocates nothing; calls on one GPU
        must not overlap)."""
        g = self.geo
        n = 0 if records is None else _batch(records, "records")
        p = _dev_ptr(records, "records", (n, g.n_heads_v, g.d, g.d), _F32, self._device)
        _check(_lib().stq_calibrate_static(ctypes.byref(self.c_state), p, n, flags,
                                           _stream(stream, self._device)), "stq_calibrate_static")

    def calibrate_impact(self, q, k, alpha, beta, flags: int, stream=None, gate=None):
        """Accumulate row impact over one step's samples (q, k [B][Hk][d], alpha,
        beta [B][Hv]); CAL_RESET / CAL_FINALIZE as in stq_calibrate_impact.
        With gate [B][Hv][d] (logical rows) the row gate replaces alpha
        (stq_calibrate_impact_gated)."""
        g, dv = self.geo, self._device
        if q is None:
            B, dt = 0, F32
        else:
            B = _batch(q, "q")
            if q.dtype not in _FLOAT_IN or k is None or k.dtype != q.dtype:
                raise ValueError("q and k must share one dtype, float32 or bfloat16")
            dt = BF16 if q.dtype == torch.bfloat16 else F32
        gated = gate is not None
        pq, pk, pr, pb = _dev_ptrs(
            (q, "q", (B, g.n_heads_k, g.d), _FLOAT_IN), (k, "k", (B, g.n_heads_k, g.d), _FLOAT_IN),
            (gate, "gate", (B, g.n_heads_v, g.d), _F32) if gated
            else (alpha, "alpha", (B, g.n_heads_v), _F32),
            (beta, "beta", (B, g.n_heads_v), _F32), device=dv)
        if gated:
            _check(_lib().stq_calibrate_impact_gated(ctypes.byref(self.c_state), pq, pk, dt, pr,
                                                     pb, B, flags, _stream(stream, self._device)),
                   "stq_calibrate_impact_gated")
            return
        _check(_lib().stq_calibrate_impact(ctypes.byref(self.c_state), pq, pk, dt, pr, pb, B,
                                           flags, _stream(stream, self._device)), "stq_calibrate_impact")

    def set_calibration(self, c: torch.Tensor, perm: torch.Tensor, stream=None):
        """Install column factors c [Hv][d] fp32 and row order perm [Hv][d]
        int32 (stq_set_calibration)."""
        g, dv = self.geo, self._device
        pc, pp = _dev_ptrs((c, "c", (g.n_heads_v, g.d), _F32),
                           (perm, "perm", (g.n_heads_v, g.d), _I32), device=dv)
        _check(_lib().stq_set_calibration(ctypes.byref(self.c_state), pc, pp,
                                          _stream(stream, self._device)), "stq_set_calibration")

    def pack(self, S: torch.Tensor, slots: torch.Tensor | None = None, stream=None):
        """Pack fp32 states S [B][Hv][d][d] (logical rows) into slots
        (stq_pack_state)."""
        g = self.geo
        B = _batch(S, "S")
        pS, ps = _dev_ptrs((S, "S", (B, g.n_heads_v, g.d, g.d), _F32), (slots, "slots", (B,), _I32),
                           device=self._device)
        _check(_lib().stq_pack_state(ctypes.byref(self.c_state), pS, ps, B,
                                     _stream(stream, self._device)), "stq_pack_state")

    def _readout(self, q, k, v, o, o_dtype):
        """The readout buffer (allocated when o is None, in o_dtype: fp32 by
        default) and the dtype argument: the input dtype, with STQ_OUT_BF16
        when o is bf16."""
        dt = _in_dtype(q, k, v)
        B = _batch(q, "q")
        if o is None:
            o = torch.empty((B, self.geo.n_heads_v, self.geo.d),
                            dtype=o_dtype or torch.float32, device=self._device)
        if not isinstance(o, torch.Tensor) or o.dtype not in _FLOAT_IN:
            raise ValueError("o must be a float32 or bfloat16 tensor")
        if o.dtype == torch.bfloat16:
            dt |= OUT_BF16
        return o, dt

    def _step_ptrs(self, q, k, v, o, slots, **rows):
        """Checked pointers of one decode step's tensors: slots [B] int32, q, k
        [B][Hk][d], v [B][Hv][d], the per-row arguments given in `rows` (alpha,
        beta [B][Hv] fp32; gate [B][Hv][d] fp32), then o [B][Hv][d]."""
        g = self.geo
        B = _batch(q, "q")
        specs = [(slots, "slots", (B,), _I32), (q, "q", (B, g.n_heads_k, g.d), _FLOAT_IN),
                 (k, "k", (B, g.n_heads_k, g.d), _FLOAT_IN),
                 (v, "v", (B, g.n_heads_v, g.d), _FLOAT_IN)]
        for name, t in rows.items():
            if t is None:
                raise ValueError(f"{name} is required")
            shape = (B, g.n_heads_v, g.d) if name == "gate" else (B, g.n_heads_v)
            specs.append((t, name, shape, _F32))
        specs.append((o, "o", (B, g.n_heads_v, g.d), _FLOAT_IN))
        return B, _dev_ptrs(*specs, device=self._device)

    def decode_step(self, q, k, v, alpha, beta, o=None, slots=None, stream=None, o_dtype=None):
        o, dt = self._readout(q, k, v, o, o_dtype)
        B, (ps, pq, pk, pv, pa, pb, po) = self._step_ptrs(q, k, v, o, slots, alpha=alpha,
                                                         beta=beta)
        _check(_lib().stq_decode_step(ctypes.byref(self.c_state), ps, B, pq, pk, pv, dt, pa, pb,
                                      po, _stream(stream, self._device)), "stq_decode_step")
        return o

    def decode_step_into(self, dst: "State", q, k, v, alpha, beta, o=None, slots=None,
                         stream=None, o_dtype=None):
        """Decode reading this state and writing the updated one into `dst`."""
        o, dt = self._readout(q, k, v, o, o_dtype)
        B, (ps, pq, pk, pv, pa, pb, po) = self._step_ptrs(q, k, v, o, slots, alpha=alpha,
                                                         beta=beta)
        _check(_lib().stq_decode_step_into(ctypes.byref(self.c_state), ctypes.byref(dst.c_state),
                                           ps, B, pq, pk, pv, dt, pa, pb, po,
                                           _stream(stream, self._device)),
               "stq_decode_step_into")
        return o

    def decode_step_gated(self, q, k, v, gate, beta, o=None, slots=None, stream=None,
                          dst: "State | None" = None, o_dtype=None):
        """Decode with a per-key-row gate [B][Hv][d] (logical rows, fp32),
        in place or, with dst, into another state (stq_decode_step_gated)."""
        o, dt = self._readout(q, k, v, o, o_dtype)
        B, (ps, pq, pk, pv, pg, pb, po) = self._step_ptrs(q, k, v, o, slots, gate=gate,
                                                         beta=beta)
        target = self if dst is None else dst
        _check(_lib().stq_decode_step_gated(ctypes.byref(self.c_state),
                                            ctypes.byref(target.c_state), ps, B, pq, pk, pv, dt,
                                            pg, pb, po, _stream(stream, self._device)),
               "stq_decode_step_gated")
        return o

    def dequant(self, B: int | None = None, slots=None, out=None, stream=None):
        g = self.geo
        if B is None:
            B = _batch(slots, "slots") if slots is not None else g.n_slots
        if out is None:
            out = torch.empty((B, g.n_heads_v, g.d, g.d), dtype=torch.float32,
                              device=self._device)
        po, ps = _dev_ptrs((out, "out", (B, g.n_heads_v, g.d, g.d), _F32),
                           (slots, "slots", (B,), _I32), device=self._device)
        _check(_lib().stq_dequant_state(ctypes.byref(self.c_state), ps, B, po,
                                        _stream(stream, self._device)), "stq_dequant_state")
        return out


def stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Copy src's bytes into dst (same byte size, same device) on the stream
    (stq_stream_copy)."""
    ps = _dev_ptr(src, "src")
    pd = _dev_ptr(dst, "dst", device=src.device)
    if ps is None or pd is None:
        raise ValueError("src and dst are required")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, src {n}")
    _check(_lib().stq_stream_copy(ps, pd, n, _stream(stream, src.device)), "stq_stream_copy")
