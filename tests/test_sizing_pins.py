"""Sizing pins: the pages' state-memory accounting re-derived, and the same
accounting applied to this library's packed format, whose bytes come from
stq_state_bytes (STEPQuant paper: App. F.1 per-request packed pages, App. F.3
Eq. M(B, L) = W + (rB + 1) S + BLK for the reserved slots, App. C.3 "Compact
dual-axis representation").  Host only."""
from __future__ import annotations

import ctypes

import pytest

stq = pytest.importorskip("linear_attention_recurrent_rule_amd.stq")

MIB, GIB = 2 ** 20, 2 ** 30
D = 128
FP32_PER_REQUEST = 150_994_944    # App. F.1: FP32 recurrent state per request
PACKED_PER_REQUEST = 29_999_104   # App. F.1: the 6-bit packed pages per request
RESERVED_COMPACT = 30_015_488     # App. F.3: compact state incl. pivot scale slots
CONV_STATE = 2_949_120            # App. F.3: the unchanged convolution state
SLOTS_PER_REQUEST = 3 + 2         # App. F.3: radix-cache slots + overlap tracking
SENTINEL = 1                      # App. F.3: one global sentinel slot


def _reserved(B: int, per_slot: int) -> int:
    """The state term of M(B, L): (r B + 1) S, with r = 5 slots per request."""
    return (SLOTS_PER_REQUEST * B + SENTINEL) * per_slot


def _per_unit_bytes(n8: int, fmt=stq.FMT_MIXED48) -> float:
    """Bytes per (slot, head) of this library's state: the growth of
    stq_state_bytes from 256 to 512 slots (the per-head calibration arrays
    and the 256-byte rounding cancel)."""
    hv = 32

    def size(n_slots):
        d_ = stq.Desc(n_slots, hv, 16, D, D, n8, fmt, 0, 0)
        return stq.lib().stq_state_bytes(ctypes.byref(d_))

    grow = size(512) - size(256)
    assert grow > 0
    return grow / (256 * hv)


def test_pages_per_request_accounting():
    # the FP32 figure is whole 128 x 128 fp32 matrices: 2304 of them, 144 MiB
    n_mat, rem = divmod(FP32_PER_REQUEST, D * D * 4)
    assert rem == 0 and n_mat == 2304 and FP32_PER_REQUEST == 144 * MIB
    assert round(PACKED_PER_REQUEST / MIB, 3) == 28.609
    assert round(FP32_PER_REQUEST / PACKED_PER_REQUEST, 2) == 5.03
    assert round(100 * (1 - PACKED_PER_REQUEST / FP32_PER_REQUEST), 2) == 80.13


def test_pages_reserved_pool_at_64_requests():
    per_slot = RESERVED_COMPACT + CONV_STATE
    assert per_slot == 31.4375 * MIB
    assert round(_reserved(64, per_slot) / GIB, 2) == 9.85
    fp32_slot = FP32_PER_REQUEST + CONV_STATE
    assert round(_reserved(64, fp32_slot) / GIB, 2) == 46.02


def test_library_format_bits_and_the_same_accounting():
    six = _per_unit_bytes(64)    # 64 int8 rows + 64 int4 rows + fp32 row factors
    four5 = _per_unit_bytes(16)  # 16 int8 rows + 112 int4 rows + fp32 row factors
    assert six == 64 * D + 64 * D // 2 + 4 * D == 12_800
    assert four5 == 16 * D + 112 * D // 2 + 4 * D == 9_728
    assert 8 * six / (D * D) == 6.25 and 8 * four5 / (D * D) == 4.75
    fp32 = _per_unit_bytes(0, stq.FMT_FP32)
    assert fp32 == D * D * 4
    n_mat = FP32_PER_REQUEST // (D * D * 4)
    ours6, ours45 = n_mat * six, n_mat * four5
    assert n_mat * fp32 == FP32_PER_REQUEST
    assert ours6 == 29_491_200 and ours45 == 22_413_312
    assert round(FP32_PER_REQUEST / ours6, 2) == 5.12
    assert round(FP32_PER_REQUEST / ours45, 2) == 6.74
    # 6.25 bits against the pages' 29,999,104 B: ours holds fp32 row factors and
    # no pivot rows; the pages' adds FP16 scales and pivots on about 6 bits
    assert ours6 < PACKED_PER_REQUEST
    # the F.3 reservation at B = 64 with this format in place of the compact one
    assert round(_reserved(64, ours6 + CONV_STATE) / GIB, 2) == 9.70
    assert round(_reserved(64, ours45 + CONV_STATE) / GIB, 2) == 7.58


def test_compact_representation_bits():
    """App. C.3 "Compact dual-axis representation": FP16 row and column
    scales cost 16 (dk + dv) / (dk dv) = 0.25 bits per value at 128 x 128;
    the four-bit packed count of 21,804,032 B per request is 4.6209 bits per
    value and 6.9251x below FP32; the KDA cost adds 0.30 bits (two FP16 scale
    vectors and 512 of 81,920 rows at 16 instead of 8 bits).  This library's
    scales are an fp32 factor per key row (0.25 bits per value) and per-head
    column factors shared by all slots (none per slot)."""
    assert 16 * (D + D) / (D * D) == 0.25
    four_bit = 21_804_032
    values = FP32_PER_REQUEST // 4
    assert round(8 * four_bit / values, 4) == 4.6209
    assert round(FP32_PER_REQUEST / four_bit, 4) == 6.9251
    assert round(16 / 128 + 16 / 128 + 512 / 81920 * (16 - 8), 2) == 0.30
    for nominal, table in ((6, 6.300), (4, 4.300)):
        assert round(nominal + 0.30, 3) == table
    six = _per_unit_bytes(64)
    row_factor_bits = 8 * 4 * D / (D * D)
    assert row_factor_bits == 0.25 and 8 * six / (D * D) - row_factor_bits == 6.0
