"""The benchmark's byte accounting (CPU): the algorithmic bytes per state
update that the roofline fraction divides by, checked against sizes worked
out by hand from the layout (codes of n8 8-bit rows and d - n8 4-bit rows,
one fp32 row factor per row, read once and written once; q and k once per
key head, v, the gate and beta once per value head, o written once), and the
source hash that ties recorded counters to the kernel they were taken on."""
from __future__ import annotations

import pytest

import bench

UNITS = 1024 * 32  # B = 1024 sequences x 32 value heads


@pytest.mark.parametrize("fmt,n8,per_unit", [
    ("mixed", 64, 2 * (64 * 128 + 64 * 64 + 4 * 128) + 1032),    # 6-bit mix: 26,632 B
    ("mixed", 16, 2 * (16 * 128 + 112 * 64 + 4 * 128) + 1032),   # 4.5-bit mix: 20,488 B
    ("int8row", 128, 2 * (128 * 128 + 4 * 128) + 1032),          # 34,824 B
    ("fp32", 0, 2 * 4 * 128 * 128 + 1032),                       # 132,104 B
    ("refit", 64, 2 * (64 * 128 + 64 * 64 + 8 * 128) + 1032),    # + the state's own c
])
def test_bytes_per_update_at_serving_shape(fmt, n8, per_unit):
    # 1,032 B of vectors: q and k 256 B each shared by two value heads, v 256 B,
    # alpha and beta 4 B each, o 512 B
    assert bench.algorithmic_bytes(fmt, 1024, 32, 16, 128, n8, 2) == UNITS * per_unit


def test_headline_launch_bytes():
    assert bench.algorithmic_bytes("mixed", 1024, 32, 16, 128, 64, 2) == 872_677_376


def test_gate_and_readout_variants():
    base = bench.algorithmic_bytes("mixed", 1024, 32, 16, 128, 64, 2)
    # a per-key-row fp32 gate (512 B) replaces the 4 B alpha
    assert bench.algorithmic_bytes("mixed", 1024, 32, 16, 128, 64, 2, gated=True) == base + UNITS * 508
    # a bf16 readout writes 256 B instead of 512 B
    assert bench.algorithmic_bytes("mixed", 1024, 32, 16, 128, 64, 2, out_el=2) == base - UNITS * 256


def test_small_workloads():
    # small_mixed: fp32 q, k, v at d = 64, no sharing of key heads
    assert bench.algorithmic_bytes("mixed", 8, 4, 4, 64, 32, 4) == 8 * 4 * (2 * 3328 + 1032)
    # tiny: d = 16, all rows 8-bit
    assert bench.algorithmic_bytes("mixed", 1, 1, 1, 16, 16, 4) == 904


def test_source_hash_ignores_comments_only():
    code = "int f(int x) {\n    return x + 1; // add one\n}\n"
    same = "/* header */\nint f(int x) {\n\n    return x + 1;\n}\n"
    other = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(code, ".hip") == bench._code_only(same, ".hip")
    assert bench._code_only(code, ".hip") != bench._code_only(other, ".hip")
    py = 'def g():\n    """doc"""\n    # note\n    return 1\n'
    assert bench._code_only(py, ".py") == bench._code_only("def g():\n    return 1\n", ".py")
