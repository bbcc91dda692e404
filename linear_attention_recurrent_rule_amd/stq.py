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
           "stq_calibrate_retention", "stq_allocate", "stq_set_alloc_layout")


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
        lib.stq_dequant_state.argtypes = [ctypes.POINTER(CState), P, I32, P, P]
        lib.stq_stream_copy.argtypes = [P, P, SZ, P]
        lib.stq_status_str.argtypes = [I32]
        lib.stq_status_str.restype = ctypes.c_char_p
        lib.stq_abi_version.restype = I32
        for name in ("stq_alloc_state", "stq_calibrate", "stq_calibrate_impact",
                     "stq_calibrate_impact_gated", "stq_set_calibration",
                     "stq_pack_state", "stq_decode_step", "stq_decode_step_into",
                     "stq_decode_step_gated", "stq_dequant_state", "stq_stream_copy",
                     "stq_calibrate_retention", "stq_allocate", "stq_set_alloc_layout"):
            getattr(lib, name).restype = I32
        _LIB = lib
    return _LIB


def lib():
    """The loaded libstq.so (raises ImportError if it has not been built)."""
    return _lib()


def _check(status: int, where: str):
    if status != STQ_OK:
        raise StqError(status, where)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _in_dtype(q, k, v) -> int:
    if q.dtype == torch.float32:
        dt = F32
    elif q.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise ValueError("q, k, v must be float32 or bfloat16")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    return dt


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
        self.c_state = CState()
        _check(_lib().stq_alloc_state(ctypes.byref(self.desc), _dev_ptr(self.buffer, "buffer"),
                                      nbytes, _stream(stream), ctypes.byref(self.c_state)),
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
        src = gate if gate is not None else alpha
        B = 0 if src is None else int(src.shape[0])
        _check(_lib().stq_calibrate_retention(ctypes.byref(self.c_state), _dev_ptr(alpha, "alpha"),
                                              _dev_ptr(gate, "gate"), B, flags, _stream(stream)),
               "stq_calibrate_retention")

    def allocate(self, horizon: int, candidates: int = 0, stream=None):
        """Pivots and row widths from the calibration statistics (stq_allocate)."""
        _check(_lib().stq_allocate(ctypes.byref(self.c_state), int(horizon), int(candidates),
                                   _stream(stream)), "stq_allocate")

    def set_alloc_layout(self, counts, c: torch.Tensor, perm: torch.Tensor, stream=None):
        """Install class counts [Hv][5] (host array), c and perm (device)."""
        import numpy as np
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        _check(_lib().stq_set_alloc_layout(ctypes.byref(self.c_state), cnt.ctypes.data,
                                           _dev_ptr(c, "c"), _dev_ptr(perm, "perm"),
                                           _stream(stream)), "stq_set_alloc_layout")

    @property
    def calibrated(self) -> bool:
        return bool(self.c_state.calibrated)

    # -- entry points --
    def calibrate(self, records: torch.Tensor | None, flags: int, stream=None):
        n = 0 if records is None else int(records.shape[0])
        _check(_lib().stq_calibrate(ctypes.byref(self.c_state), _dev_ptr(records, "records"),
                                    n, flags, _stream(stream)), "stq_calibrate")

    def calibrate_impact(self, q, k, alpha, beta, flags: int, stream=None, gate=None):
        """Accumulate row impact over one step's samples (q, k [B][Hk][d], alpha,
        beta [B][Hv]); CAL_RESET / CAL_FINALIZE as in stq_calibrate_impact.
        With gate [B][Hv][d] (logical rows) the row gate replaces alpha
        (stq_calibrate_impact_gated)."""
        if q is None:
            B, dt = 0, F32
        else:
            B = int(q.shape[0])
            dt = BF16 if q.dtype == torch.bfloat16 else F32
        if gate is not None:
            _check(_lib().stq_calibrate_impact_gated(
                ctypes.byref(self.c_state), _dev_ptr(q, "q"), _dev_ptr(k, "k"), dt,
                _dev_ptr(gate, "gate"), _dev_ptr(beta, "beta"), B, flags, _stream(stream)),
                "stq_calibrate_impact_gated")
            return
        _check(_lib().stq_calibrate_impact(ctypes.byref(self.c_state), _dev_ptr(q, "q"),
                                           _dev_ptr(k, "k"), dt, _dev_ptr(alpha, "alpha"),
                                           _dev_ptr(beta, "beta"), B, flags, _stream(stream)),
               "stq_calibrate_impact")

    def set_calibration(self, c: torch.Tensor, perm: torch.Tensor, stream=None):
        _check(_lib().stq_set_calibration(ctypes.byref(self.c_state), _dev_ptr(c, "c"),
                                          _dev_ptr(perm, "perm"), _stream(stream)),
               "stq_set_calibration")

    def pack(self, S: torch.Tensor, slots: torch.Tensor | None = None, stream=None):
        B = int(S.shape[0])
        _check(_lib().stq_pack_state(ctypes.byref(self.c_state), _dev_ptr(S, "S"),
                                     _dev_ptr(slots, "slots"), B, _stream(stream)),
               "stq_pack_state")

    def _readout(self, q, k, v, o, o_dtype):
        """The readout buffer (allocated when o is None, in o_dtype: fp32 by
        default) and the dtype argument: the input dtype, with STQ_OUT_BF16
        when o is bf16."""
        dt = _in_dtype(q, k, v)
        if o is None:
            o = torch.empty((int(q.shape[0]), self.geo.n_heads_v, self.geo.d),
                            dtype=o_dtype or torch.float32, device=q.device)
        if o.dtype == torch.bfloat16:
            dt |= OUT_BF16
        elif o.dtype != torch.float32:
            raise ValueError("o must be float32 or bfloat16")
        return o, dt

    def decode_step(self, q, k, v, alpha, beta, o=None, slots=None, stream=None, o_dtype=None):
        B = int(q.shape[0])
        o, dt = self._readout(q, k, v, o, o_dtype)
        _check(_lib().stq_decode_step(ctypes.byref(self.c_state), _dev_ptr(slots, "slots"), B,
                                      _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), dt,
                                      _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                      _dev_ptr(o, "o"), _stream(stream)), "stq_decode_step")
        return o

    def decode_step_into(self, dst: "State", q, k, v, alpha, beta, o=None, slots=None,
                         stream=None, o_dtype=None):
        """Decode reading this state and writing the updated one into `dst`."""
        B = int(q.shape[0])
        o, dt = self._readout(q, k, v, o, o_dtype)
        _check(_lib().stq_decode_step_into(ctypes.byref(self.c_state), ctypes.byref(dst.c_state),
                                           _dev_ptr(slots, "slots"), B, _dev_ptr(q, "q"),
                                           _dev_ptr(k, "k"), _dev_ptr(v, "v"), dt,
                                           _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                           _dev_ptr(o, "o"), _stream(stream)),
               "stq_decode_step_into")
        return o

    def decode_step_gated(self, q, k, v, gate, beta, o=None, slots=None, stream=None,
                          dst: "State | None" = None, o_dtype=None):
        """Decode with a per-key-row gate [B][Hv][d] (logical rows, fp32),
        in place or, with dst, into another state (stq_decode_step_gated)."""
        B = int(q.shape[0])
        o, dt = self._readout(q, k, v, o, o_dtype)
        target = self if dst is None else dst
        _check(_lib().stq_decode_step_gated(ctypes.byref(self.c_state),
                                            ctypes.byref(target.c_state),
                                            _dev_ptr(slots, "slots"), B, _dev_ptr(q, "q"),
                                            _dev_ptr(k, "k"), _dev_ptr(v, "v"), dt,
                                            _dev_ptr(gate, "gate"), _dev_ptr(beta, "beta"),
                                            _dev_ptr(o, "o"), _stream(stream)),
               "stq_decode_step_gated")
        return o

    def dequant(self, B: int | None = None, slots=None, out=None, stream=None):
        if B is None:
            B = int(slots.shape[0]) if slots is not None else self.geo.n_slots
        if out is None:
            out = torch.empty((B, self.geo.n_heads_v, self.geo.d, self.geo.d),
                              dtype=torch.float32, device=self.buffer.device)
        _check(_lib().stq_dequant_state(ctypes.byref(self.c_state), _dev_ptr(slots, "slots"), B,
                                        _dev_ptr(out, "S_out"), _stream(stream)),
               "stq_dequant_state")
        return out


def stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    n = src.numel() * src.element_size()
    _check(_lib().stq_stream_copy(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"), n,
                                  _stream(stream)), "stq_stream_copy")
