"""The LDS-poisoning debug build really fills LDS: compiled with
EXATTN_POISON_LDS, a kernel source gains the fill stores (ds_write) and the
barrier after them; compiled without it, its device code has neither.  (The
GPU test that runs the debug build against the ordinary one is only as good
as this.)"""

import os
import subprocess

import pytest

from exact_attention_69_amd import build


def device_asm(tmp_path, src, extra):
    out = tmp_path / ("poison.s" if extra else "plain.s")
    cmd = [build.hipcc()] + build.common_flags() + list(extra) + ["-S", "--cuda-device-only", src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_poison_macro_adds_lds_fill_and_barrier(tmp_path):
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    src = os.path.join(build.CSRC, "fp8.hip")
    plain = device_asm(tmp_path, src, ())
    poison = device_asm(tmp_path, src, ("-DEXATTN_POISON_LDS",))
    count = lambda s, op: sum(1 for line in s.splitlines() if line.strip().startswith(op))
    # fp8.hip holds the quantiser (one LDS array) and the FP8 forward (two),
    # each instantiated for d = 64 and 128
    assert count(poison, "ds_write") > count(plain, "ds_write")
    assert count(poison, "s_barrier") >= count(plain, "s_barrier") + 4
