"""Host check of the ragged decode's per-slot load descriptors.

The descriptors are written with the layout (stq_api.cpp build_layout and the
initial-layout kernel both call slot_descs_128 from stq_internal.h).  The
check program compiles that header for the host and compares every lane's
chunk offsets with the per-class row layout for 20,000 seeded class-count
vectors (tests/native/slot_desc_check.cpp).
"""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc (ROCm) not installed")
def test_slot_descriptors_match_class_layout(tmp_path):
    exe = tmp_path / "slot_desc_check"
    subprocess.run([_hipcc(), "-O2", "-std=c++17", f"-I{ROOT / 'include'}",
                    f"-I{ROOT / 'linear_attention_recurrent_rule_amd' / 'csrc'}",
                    str(ROOT / "tests" / "native" / "slot_desc_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    assert out.startswith("ok:"), out
